"""The C ABI on the CPU: the library loads, exports every entry point include/ra.h
declares, and rejects bad arguments with the documented codes before touching the GPU
(no call here gets as far as a launch)."""

import ctypes
import os
import re

import pytest

from blockwise_ring_attention_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "ra.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(B.EXPORTED)


def _declared_signatures():
    """{name: [parameter type strings]} from the prototypes in include/ra.h."""
    text = open(os.path.join(ROOT, "include", "ra.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    sigs = {}
    for m in re.finditer(r"\b(ra_\w+)\s*\(([^)]*)\)\s*;", text):
        params = [p.strip() for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        sigs[m.group(1)] = [re.sub(r"\s*\b\w+$", "", p).strip() for p in params]
    return sigs


def _ctype_for(c_type: str):
    if "*" in c_type:
        return ctypes.c_void_p
    return {"int": ctypes.c_int, "long long": ctypes.c_longlong}[c_type]


def test_binding_argtypes_match_the_header(ra_lib):
    """Every ctypes prototype in the binding has the header's parameter count and types,
    so a change on one side of the boundary cannot silently shift arguments."""
    lib = B.load()
    sigs = _declared_signatures()
    assert sorted(sigs) == sorted(B.EXPORTED)
    for name, params in sigs.items():
        fn = getattr(lib, name)
        assert list(fn.argtypes) == [_ctype_for(p) for p in params], name


def test_library_exports_every_declared_symbol(ra_lib):
    for name in _declared_functions():
        assert hasattr(ra_lib, name), name
        assert ctypes.cast(getattr(ra_lib, name), ctypes.c_void_p).value


def test_version(ra_lib):
    assert B.version() == 300


FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced (every call below fails its checks)


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, batch=1, hq=4, hkv=2, nq=64, nkv=64, d=128, c=4, rank=1,
             causal=1, zigzag=1, t0=0, t1=4, dtype=B.RA_BF16)
    a.update(kw)
    return B.ra_rank_forward(a["q"], a["k"], a["v"], a["out"], a["lse"], a["batch"], a["hq"], a["hkv"], a["nq"],
                             a["nkv"], a["d"], a["c"], a["rank"], a["causal"], a["zigzag"], a["t0"], a["t1"],
                             a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), B.RA_ERR_ARG),
    (dict(batch=-1), B.RA_ERR_ARG),
    (dict(hq=0), B.RA_ERR_ARG),
    (dict(hq=6, hkv=4), B.RA_ERR_ARG),
    (dict(c=0, rank=0, t1=0), B.RA_ERR_ARG),
    (dict(rank=4), B.RA_ERR_ARG),
    (dict(rank=-1), B.RA_ERR_ARG),
    (dict(t0=3, t1=2), B.RA_ERR_ARG),
    (dict(t1=5), B.RA_ERR_ARG),
    (dict(d=96), B.RA_ERR_UNSUPPORTED),
    (dict(d=256), B.RA_ERR_UNSUPPORTED),
    (dict(dtype=B.RA_F32, d=12), B.RA_ERR_UNSUPPORTED),
    (dict(dtype=B.RA_F32, d=136), B.RA_ERR_UNSUPPORTED),
    (dict(nkv=32), B.RA_ERR_SHAPE),
    (dict(nq=63, nkv=63), B.RA_ERR_SHAPE),
    (dict(c=1 << 16, rank=0, t1=1, nq=1 << 15, nkv=1 << 15), B.RA_ERR_SHAPE),
    (dict(c=1, rank=0, t1=1, nq=1 << 24, nkv=1 << 24), B.RA_ERR_SHAPE),   # 4 GiB K slab per head
    (dict(q=0), B.RA_ERR_ARG),
    (dict(out=0), B.RA_ERR_ARG),
    (dict(k=0), B.RA_ERR_ARG),
    (dict(q=FAKE + 8), B.RA_ERR_ALIGN),
    (dict(v=FAKE + 2), B.RA_ERR_ALIGN),
    (dict(lse=FAKE + 2), B.RA_ERR_ALIGN),
])
def test_forward_argument_errors(ra_lib, kw, code):
    assert _fwd(**kw) == code
    assert B.last_error() != ""


def _fwd_doc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, doc=FAKE, out=FAKE, lse=FAKE, batch=1, hq=4, hkv=2, nq=64, nkv=64, d=128, c=4,
             rank=1, zigzag=1, t0=0, t1=4, dtype=B.RA_BF16)
    a.update(kw)
    return B.ra_rank_forward_doc(a["q"], a["k"], a["v"], a["doc"], a["out"], a["lse"], a["batch"], a["hq"], a["hkv"],
                                 a["nq"], a["nkv"], a["d"], a["c"], a["rank"], a["zigzag"], a["t0"], a["t1"],
                                 a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(doc=0), B.RA_ERR_ARG),
    (dict(doc=FAKE + 2), B.RA_ERR_ALIGN),
    (dict(rank=4), B.RA_ERR_ARG),
    (dict(nkv=32), B.RA_ERR_SHAPE),          # always causal: nq == nkv
    (dict(nq=63, nkv=63), B.RA_ERR_SHAPE),   # zigzag needs an even nkv
    (dict(d=96), B.RA_ERR_UNSUPPORTED),
    (dict(q=FAKE + 8), B.RA_ERR_ALIGN),
])
def test_forward_doc_argument_errors(ra_lib, kw, code):
    assert _fwd_doc(**kw) == code
    assert B.last_error() != ""


def test_forward_doc_empty_is_a_noop(ra_lib):
    assert _fwd_doc(batch=0, q=0, k=0, v=0, doc=0, out=0, lse=0) == B.RA_OK
    assert _fwd_doc(nq=0, nkv=0, q=0, k=0, v=0, doc=0, out=0, lse=0) == B.RA_OK


def _fwd_acc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, doc=0, out=FAKE, lse=FAKE, batch=1, hq=4, hkv=2, nq=64, nkv=64, d=128, c=4,
             rank=1, causal=1, zigzag=1, t0=0, t1=4, dtype=B.RA_BF16, out_dtype=None)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    return B.ra_rank_forward_accumulate(a["q"], a["k"], a["v"], a["doc"], a["out"], a["lse"], a["batch"], a["hq"],
                                        a["hkv"], a["nq"], a["nkv"], a["d"], a["c"], a["rank"], a["causal"],
                                        a["zigzag"], a["t0"], a["t1"], a["dtype"], od, None)


@pytest.mark.parametrize("kw,code", [
    (dict(lse=0), B.RA_ERR_ARG),                    # the running lse is required
    (dict(lse=0, doc=FAKE), B.RA_ERR_ARG),
    (dict(doc=FAKE, causal=0), B.RA_ERR_ARG),       # the document mask is causal
    (dict(doc=FAKE + 2), B.RA_ERR_ALIGN),
    (dict(lse=FAKE + 2), B.RA_ERR_ALIGN),
    (dict(t0=2, t1=1), B.RA_ERR_ARG),
    (dict(nkv=32), B.RA_ERR_SHAPE),
    (dict(d=96), B.RA_ERR_UNSUPPORTED),
    (dict(out=0), B.RA_ERR_ARG),
    (dict(out_dtype=7), B.RA_ERR_ARG),
    (dict(dtype=B.RA_F32, d=64, out_dtype=B.RA_BF16), B.RA_ERR_ARG),   # fp32 inputs need an fp32 out
    (dict(out_dtype=B.RA_F32, out=FAKE + 8), B.RA_ERR_ALIGN),
])
def test_forward_accumulate_argument_errors(ra_lib, kw, code):
    assert _fwd_acc(**kw) == code
    assert B.last_error() != ""


# distinct 16-byte aligned fake addresses, 1 MiB apart (larger than any tensor below)
QA, KA, VA, OA, LA, DA = (0x100000 * i for i in range(1, 7))


@pytest.mark.parametrize("kw", [
    dict(out=QA),                  # out is q
    dict(out=KA + 4096),           # out starts inside k_blocks
    dict(lse=VA + 65536),          # lse inside v_blocks
    dict(out=QA + 32768),          # out starts inside q
    dict(lse=OA + 1024),           # lse inside out
    dict(out=LA - 16),             # out ends inside lse
])
def test_forward_outputs_must_not_overlap_inputs(ra_lib, kw):
    a = dict(q=QA, k=KA, v=VA, out=OA, lse=LA)
    a.update(kw)
    assert _fwd(**a) == B.RA_ERR_ARG
    assert "overlap" in B.last_error()
    assert _fwd_acc(**a) == B.RA_ERR_ARG
    assert _fwd_acc(**a, out_dtype=B.RA_F32) == B.RA_ERR_ARG


def test_forward_doc_outputs_must_not_overlap_doc_start(ra_lib):
    assert _fwd_doc(q=QA, k=KA, v=VA, doc=DA, out=DA + 512, lse=LA) == B.RA_ERR_ARG
    assert _fwd_doc(q=QA, k=KA, v=VA, doc=DA, out=OA, lse=DA - 16) == B.RA_ERR_ARG
    assert "overlap" in B.last_error()


def test_forward_accumulate_empty_is_a_noop(ra_lib):
    assert _fwd_acc(batch=0, q=0, k=0, v=0, out=0, lse=0) == B.RA_OK
    assert _fwd_acc(nq=0, nkv=0, q=0, k=0, v=0, out=0, lse=0, causal=0) == B.RA_OK


def test_forward_empty_is_a_noop(ra_lib):
    assert _fwd(nq=0, nkv=0, q=0, k=0, v=0, out=0, lse=0, causal=0) == B.RA_OK
    assert _fwd(batch=0, q=0, k=0, v=0, out=0, lse=0) == B.RA_OK


def _merge(**kw):
    a = dict(oa=FAKE, la=FAKE, ob=FAKE, lb=FAKE, o=FAKE, l=FAKE, rows=10, d=128, dtype=B.RA_BF16)
    a.update(kw)
    return B.ra_merge(a["oa"], a["la"], a["ob"], a["lb"], a["o"], a["l"], a["rows"], a["d"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), B.RA_ERR_ARG),
    (dict(rows=-1), B.RA_ERR_ARG),
    (dict(d=12), B.RA_ERR_UNSUPPORTED),
    (dict(d=520), B.RA_ERR_UNSUPPORTED),
    (dict(ob=0), B.RA_ERR_ARG),
    (dict(l=0), B.RA_ERR_ARG),
    (dict(o=FAKE + 4), B.RA_ERR_ALIGN),
    (dict(la=FAKE + 1), B.RA_ERR_ALIGN),
])
def test_merge_argument_errors(ra_lib, kw, code):
    assert _merge(**kw) == code


def test_merge_empty_is_a_noop(ra_lib):
    assert _merge(rows=0, oa=0, la=0, ob=0, lb=0, o=0, l=0) == B.RA_OK


def test_check_raises_with_text(ra_lib):
    assert _fwd(rank=9) == B.RA_ERR_ARG
    with pytest.raises(B.RaValueError, match="rank=9"):
        B.check(B.RA_ERR_ARG, "ra_rank_forward")
    with pytest.raises(B.RaError):
        B.check(B.RA_ERR_LAUNCH, "ra_rank_forward")


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        B.load(str(tmp_path / "libra.so"))


def test_sweep_configurations_are_valid():
    """Every configuration of the GPU sweep passes the library's own argument rules, and
    the sweep spans the modes and flags it claims to."""
    from tests.test_gpu_sweep import N_CASES, _draw
    modes, flags = set(), set()
    for i in range(N_CASES):
        p = _draw(i)
        assert p["hq"] % p["hkv"] == 0 and 1 <= p["hq"] <= 32
        assert (p["dtype"] == "bf16" and p["d"] in (64, 128)) or (p["dtype"] == "f32" and p["d"] % 8 == 0
                                                                  and 8 <= p["d"] <= 128)
        assert 0 <= p["rank"] < p["c"] and 0 <= p["t0"] <= p["t1"] <= p["c"]
        assert p["n"] >= 2 and (not p["zigzag"] or p["n"] % 2 == 0)
        assert p["mode"] != "doc" or p["causal"]
        assert p["mode"] != "accumulate" or p["t1"] > p["t0"]
        modes.add(p["mode"])
        flags.add((p["causal"], p["zigzag"], p["dtype"]))
    assert modes == {"fused", "doc", "accumulate"}
    assert len(flags) >= 7


def test_ablation_libraries_export_the_boundary():
    """The design-choice comparison builds (made by the build script beside libra.so) load
    and export every entry point the header declares, so the bench can time them through
    the same calls."""
    from blockwise_ring_attention_amd.csrc import build
    for name in [*build.ABLATIONS, *build.DIAGNOSTICS]:
        path = build.ablation_path(name)
        if not os.path.exists(path):
            pytest.skip(f"{path} not built (build_ablations)")
        lib = ctypes.CDLL(path)
        for sym in _declared_functions():
            assert hasattr(lib, sym), (name, sym)


def test_timeline_registration_only_in_the_diagnostic_build(ra_lib):
    """ra_diag_timeline exists only in the diagnostic build, and rejects a buffer without
    a capacity (and the reverse) before touching the device."""
    from blockwise_ring_attention_amd.csrc import build
    assert not hasattr(ra_lib, "ra_diag_timeline")
    path = build.ablation_path("timeline")
    if not os.path.exists(path):
        pytest.skip(f"{path} not built (build_ablations)")
    lib = ctypes.CDLL(path)
    lib.ra_diag_timeline.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.ra_diag_timeline.restype = ctypes.c_int
    assert lib.ra_diag_timeline(None, 4) == -1
    assert lib.ra_diag_timeline(ctypes.c_void_p(4096), 0) == -1
    assert lib.ra_diag_timeline(ctypes.c_void_p(4096), -1) == -1


def test_plain_c_consumer_builds(tmp_path, ra_lib):
    """The boundary is usable from plain C: a C11 program including only ra.h and the HIP
    runtime API compiles with gcc and links against libra.so (it runs in the GPU tests)."""
    from tests.c_consumer import build
    assert os.path.exists(build(str(tmp_path / "ra_c_consumer")))
