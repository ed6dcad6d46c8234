"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/specverify.h declares,
and reject bad arguments with the documented status before any HIP call.
"""

import ctypes
import os
import re

import pytest

from rejection_sampling_verifier_spec_amd import api
from rejection_sampling_verifier_spec_amd.build import LIB, build_library

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "specverify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        build_library()
    return api.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("spec_verify_probs", "spec_verify_greedy", "spec_verify_ragged", "spec_verify_workspace_size",
              "spec_verify_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(declared_functions()) == sorted(api.EXPORTS)
    assert lib.spec_verify_version() == 3


def test_status_strings(lib):
    assert api.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert api.status_string(s) != "unknown status"
    assert api.status_string(7) == "unknown status"


def test_workspace_size(lib):
    # records + counters + 48-byte list entries + per-row tile counters + three fp64 and one int
    # per-tile arrays (nt = ceil(V / 2048)) + per-row {m, Z, bound, shift} + per-request marks
    # + the second lazy launch's {request, position} tasks; each part 256-aligned
    assert api.workspace_size(1, 100) == 256 * 11
    assert api.workspace_size(2048, 128256) == (2048 * 8 + 256 + 2048 * 48 + 2048 * 4
                                                + 3 * 2048 * 63 * 8 + 2048 * 63 * 4 + 2048 * 32 + 2048 * 4
                                                + 2048 * 8)
    assert lib.spec_verify_workspace_size(-1, 100) == 0
    assert lib.spec_verify_workspace_size(5, 0) == 0
    assert lib.spec_verify_workspace_size(5, (1 << 21) + 1) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation or has B == 0


def probs(lib, **kw):
    a = dict(logits=FAKE, dtype=1, q=FAKE, x=FAKE, u=FAKE, B=2, g=3, V=100, T=1.0, flags=0, out=FAKE, nacc=FAKE,
             stats=None, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.spec_verify_probs(a["logits"], a["dtype"], a["q"], a["x"], a["u"], a["B"], a["g"], a["V"], a["T"],
                                 a["flags"], a["out"], a["nacc"], a["stats"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -1),
    (dict(g=-1), -1),
    (dict(V=0), -1),
    (dict(V=(1 << 21) + 1), -2),
    (dict(dtype=7), -2),
    (dict(T=-0.5), -1),
    (dict(T=float("nan")), -1),
    (dict(T=float("inf")), -1),
    (dict(T=1e-39), -1),        # log2(e) / T beyond the fp32 range
    (dict(T=4.2e-39), -1),
    (dict(T=5e-39, B=0), 0),    # the smallest temperatures whose scale fits fp32 pass validation
    (dict(flags=0x10), -1),
    (dict(logits=None), -1),
    (dict(out=None), -1),
    (dict(nacc=None), -1),
    (dict(x=None), -1),
    (dict(u=None), -1),
    (dict(stats=FAKE, T=0.0), -1),
    (dict(ws=None), -4),
    (dict(wsb=8 * 7), -4),
    (dict(wsb=3071), -4),  # 8 rows, V=100 need 3072 bytes
    (dict(ws=ctypes.c_void_p(0x1080)), -4),
    (dict(B=0), 0),
])
def test_probs_argument_validation(lib, kw, status):
    assert probs(lib, **kw) == status


def test_greedy_and_ragged_validation(lib):
    g = lib.spec_verify_greedy
    assert g(FAKE, 1, FAKE, -1, 2, 10, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert g(FAKE, 3, FAKE, 1, 2, 10, FAKE, FAKE, FAKE, 1 << 20, None) == -2
    assert g(FAKE, 1, FAKE, 4, 2, 10, FAKE, FAKE, FAKE, 8, None) == -4
    assert g(FAKE, 1, FAKE, 0, 2, 10, FAKE, FAKE, FAKE, 0, None) == 0
    r = lib.spec_verify_ragged
    # missing cu offsets
    assert r(FAKE, 1, FAKE, FAKE, None, FAKE, 2, 5, 100, 1.0, 0, FAKE, FAKE, None, FAKE, 1 << 20, None) == -1
    assert r(FAKE, 1, FAKE, FAKE, FAKE, FAKE, 2, -1, 100, 1.0, 0, FAKE, FAKE, None, FAKE, 1 << 20, None) == -1
    assert r(FAKE, 1, FAKE, FAKE, FAKE, FAKE, 0, 0, 100, 1.0, 0, FAKE, FAKE, None, FAKE, 0, None) == 0


def filtered(lib, **kw):
    a = dict(logits=FAKE, dtype=1, q=FAKE, x=FAKE, u=FAKE, B=2, g=3, V=100, T=1.0, k=10, p=0.9, out=FAKE, nacc=FAKE,
             ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.spec_verify_probs_filtered(a["logits"], a["dtype"], a["q"], a["x"], a["u"], a["B"], a["g"], a["V"],
                                          a["T"], a["k"], a["p"], a["out"], a["nacc"], a["ws"], a["wsb"],
                                          a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(T=0.0), -1),          # greedy verification takes no filters
    (dict(T=-1.0), -1),
    (dict(p=0.0), -1),
    (dict(p=-0.5), -1),
    (dict(p=1.5), -1),
    (dict(p=float("nan")), -1),
    (dict(q=None), -1),         # the filters need q (already adjusted by the drafter)
    (dict(u=None), -1),
    (dict(V=0), -1),
    (dict(dtype=5), -2),
    (dict(ws=None), -4),
    (dict(wsb=3071), -4),
    (dict(B=0), 0),
    (dict(B=0, k=-3, p=1.0), 0),
])
def test_filtered_argument_validation(lib, kw, status):
    assert filtered(lib, **kw) == status


def test_ragged_filtered_validation(lib):
    r = lib.spec_verify_ragged_filtered
    assert r(FAKE, 1, FAKE, FAKE, None, FAKE, 2, 5, 100, 1.0, 5, 0.9, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert r(FAKE, 1, FAKE, FAKE, FAKE, FAKE, 2, 5, 100, 1.0, 5, 0.0, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert r(FAKE, 1, None, FAKE, FAKE, FAKE, 2, 5, 100, 1.0, 5, 0.9, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert r(FAKE, 1, FAKE, FAKE, FAKE, FAKE, 0, 0, 100, 1.0, 5, 0.9, FAKE, FAKE, FAKE, 0, None) == 0


def test_stream_read_validation(lib):
    """Rejected on the host before anything is launched: no result pointer, a
    size that is not a multiple of 16, a source that is not 16-byte aligned."""
    f = lib.spec_verify_stream_read
    assert f(FAKE, 16, None, None) == -1
    assert f(FAKE, 15, FAKE, None) == -1
    assert f(ctypes.c_void_p(0x1004), 16, FAKE, None) == -1
    assert f(None, 16, FAKE, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(api, "_lib", None)
    monkeypatch.setattr(api, "LIB_PATH", "/nonexistent/libspecverify.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        api.load()


def test_profile_argument_validation(lib):
    # rejected before any HIP call: no kernel selected, unknown kernel bit, bad capacity
    assert lib.spec_verify_profile_start(0, 10) == -1
    assert lib.spec_verify_profile_start(8, 10) == -1
    assert lib.spec_verify_profile_start(1, 0) == -1
    assert lib.spec_verify_profile_start(1, (1 << 20) + 1) == -1
    assert lib.spec_verify_profile_every(0) == -1
    # nothing recorded: stop reports zeros and touches no device state
    total = (ctypes.c_double * 3)(7.0, 7.0, 7.0)
    count = (ctypes.c_int32 * 3)(7, 7, 7)
    assert lib.spec_verify_profile_stop(ctypes.cast(total, ctypes.c_void_p), ctypes.cast(count, ctypes.c_void_p)) == 0
    assert list(total) == [0.0, 0.0, 0.0] and list(count) == [0, 0, 0]


def noalloc(lib, **kw):
    a = dict(logits=FAKE, dtype=1, q=FAKE, x=FAKE, u=FAKE, B=2, g=3, V=100, T=1.0, flags=0, out=FAKE, nacc=FAKE,
             stats=None, stream=None)
    a.update(kw)
    return lib.spec_verify_probs_noalloc(a["logits"], a["dtype"], a["q"], a["x"], a["u"], a["B"], a["g"], a["V"],
                                         a["T"], a["flags"], a["out"], a["nacc"], a["stats"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -1),
    (dict(g=-1), -1),
    (dict(V=0), -2),
    (dict(V=(1 << 21) + 1), -2),
    (dict(B=1200, g=7, V=128256), -4),   # more workspace than the fixed scratch holds
    (dict(B=1 << 16, g=7, V=1 << 21), -4),
    (dict(B=0), 0),
])
def test_noalloc_argument_validation(lib, kw, status):
    """Checked on the host before the scratch is set up or anything launched."""
    assert noalloc(lib, **kw) == status


def test_noalloc_scratch_limit_matches_the_header(lib):
    text = open(HEADER).read()
    m = re.search(r"#define SV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == api.SV_NOALLOC_SCRATCH_BYTES
    # the largest workloads the bench measures fit (workspace of each)
    for rows, V in ((256 * 8, 128256), (2819, 152064), (1024 * 5, 128256), (64 * 6, 32000)):
        assert api.workspace_size(rows, V) <= api.SV_NOALLOC_SCRATCH_BYTES
