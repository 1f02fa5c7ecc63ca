"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before touching the device.  CPU only: no call here
reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from sparse_attention_video_flash_amd import svgear as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "svgear.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(svgear_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = sv.load()
    names = _declared()
    assert set(names) == set(sv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.svgear_version() == 20000


def test_status_strings():
    assert sv.status_string(0) == "ok"
    for c in range(-9, 0):
        assert sv.status_string(c) != "unknown status"


def _shape(**kw):
    base = dict(H=2, Nq=1000, Nk=900, d=128, Cq=10, Ck=30, iters=10, dtype=sv.BF16)
    base.update(kw)
    return sv.make_shape(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), sv.E_SHAPE), (dict(Nq=0), sv.E_SHAPE), (dict(Nk=(1 << 20) + 1), sv.E_SHAPE),
    (dict(d=96), sv.E_SHAPE), (dict(Cq=0), sv.E_SHAPE), (dict(Cq=1001), sv.E_SHAPE),
    (dict(Ck=901), sv.E_SHAPE), (dict(Ck=5000, Nk=6000), sv.E_SHAPE), (dict(iters=0), sv.E_SHAPE),
    (dict(dtype=7), sv.E_DTYPE)])
def test_workspace_bytes_rejects_bad_shapes(kw, code):
    n = ctypes.c_size_t(0)
    rc = sv.load().svgear_workspace_bytes(ctypes.byref(_shape(**kw)), ctypes.byref(n))
    assert rc == code


def test_workspace_grows_with_problem():
    a = sv.workspace_bytes(_shape())
    b = sv.workspace_bytes(_shape(H=4))
    c = sv.workspace_bytes(_shape(Nq=2000, Nk=1800))
    assert 0 < a < b and a < c
    assert a % 256 == 0


FAKE = 1 << 40  # 256-aligned, never dereferenced: every call below fails validation first


def _cluster(shape, side=0, X=FAKE, V=None, init=FAKE, flags=0, ws=FAKE, ws_bytes=None, vbar=None,
             Vp=None, labels=FAKE):
    if ws_bytes is None:
        ws_bytes = 1  # too small on purpose unless a test overrides
    return sv.load().svgear_cluster(ctypes.byref(shape), side, X, V, init, flags, labels, FAKE, vbar, FAKE,
                                    FAKE, FAKE, FAKE, FAKE, Vp, ws, ws_bytes, None)


def test_cluster_validation_order():
    s = _shape()
    assert _cluster(s, X=None) == sv.E_NULL
    assert _cluster(s, X=FAKE + 8) == sv.E_ALIGN
    assert _cluster(s, side=2) == sv.E_ARG
    assert _cluster(s, flags=64) == sv.E_ARG
    assert _cluster(s, init=None) == sv.E_NULL
    assert _cluster(s, side=1) == sv.E_NULL               # V, vbar, Vp missing on the key side
    assert _cluster(s, side=0, V=FAKE) == sv.E_ARG          # V given on the query side
    assert _cluster(s, ws=None, ws_bytes=10 ** 12) == sv.E_NULL
    assert _cluster(s, ws=FAKE + 16, ws_bytes=10 ** 12) == sv.E_ALIGN
    assert _cluster(s) == sv.E_WORKSPACE
    assert _cluster(s, ws_bytes=sv.workspace_bytes(s) - 1) == sv.E_WORKSPACE


def test_probe_route_attention_forward_validation():
    L = sv.load()
    s = _shape()
    big = sv.workspace_bytes(s)
    r = ctypes.byref
    assert L.svgear_probe(r(s), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, big, None) == sv.E_NULL
    assert L.svgear_probe(r(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, sv.DEBUG_EPS, FAKE, None, FAKE, big,
                          None) == sv.E_NULL
    assert L.svgear_probe(r(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, sv.LABELS_GIVEN, FAKE, None, FAKE,
                          big, None) == sv.E_ARG
    assert L.svgear_probe(r(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, 5, None) \
        == sv.E_WORKSPACE
    for rho in (-0.1, 1.5, float("nan")):
        assert L.svgear_route(r(s), rho, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == sv.E_RHO
    assert L.svgear_route(r(s), 0.5, FAKE, None, FAKE, FAKE, FAKE, FAKE, big, None) == sv.E_NULL
    assert L.svgear_route(r(s), 0.5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 17, None) == sv.E_WORKSPACE
    assert L.svgear_attention(r(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, big,
                              None) == sv.E_NULL
    assert L.svgear_attention(r(s), FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big,
                              None) == sv.E_ALIGN
    assert L.svgear_forward(r(s), 2.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, big, None) == sv.E_RHO
    assert L.svgear_forward(r(s), 0.2, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 0, FAKE, big, None) == sv.E_NULL
    assert L.svgear_forward(r(s), 0.2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, big - 256, None) \
        == sv.E_WORKSPACE
    # forward takes SVGEAR_DEBUG_SYNC only
    for flags in (sv.LABELS_GIVEN, sv.DEBUG_EPS, sv.PROBE_LOGIT, 1 << 10):
        assert L.svgear_forward(r(s), 0.2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, flags, FAKE, big, None) \
            == sv.E_ARG
    bad = _shape(d=32)
    assert L.svgear_forward(r(bad), 0.2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, big, None) == sv.E_SHAPE


def test_route_rows_and_probe_variant_validation():
    L = sv.load()
    s = _shape()
    big = sv.workspace_bytes(s)
    r = ctypes.byref
    for rho in (-0.1, 1.5, float("nan")):
        assert L.svgear_route_rows(r(s), rho, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == sv.E_RHO
    assert L.svgear_route_rows(r(s), 0.5, FAKE, FAKE, None, FAKE, FAKE, FAKE, big, None) == sv.E_NULL
    assert L.svgear_route_rows(r(s), 0.5, FAKE, FAKE, FAKE, FAKE + 2, FAKE, FAKE, big, None) == sv.E_ALIGN
    assert L.svgear_route_rows(r(s), 0.5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 17, None) == sv.E_WORKSPACE
    # the score ratio combines with neither the logit-only estimate nor the per-key debug output
    for flags in (sv.PROBE_SCORE | sv.PROBE_LOGIT, sv.PROBE_SCORE | sv.DEBUG_EPS, 32):
        assert L.svgear_probe(r(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, flags, FAKE, FAKE, FAKE, big,
                              None) == sv.E_ARG


@pytest.mark.parametrize("H", [1, 40])
def test_workspace_at_the_maximum_shape_scales_with_the_inputs(H):
    """At the largest declared shape (N = 2^20 tokens, 4096 clusters per side)
    the workspace stays within twice the bytes of Q, K and V themselves (it
    holds their reordered copies) plus one routed-key row list of N entries per
    attention workgroup (256), so the declared limits fit one device."""
    N, C, d = 1 << 20, 4096, 128
    for dtype, eb in ((sv.BF16, 2), (sv.F32, 4)):
        s = sv.make_shape(H, N, N, d, C, C, 10, dtype)
        inputs = 3 * H * N * d * eb
        assert sv.workspace_bytes(s) <= 2 * inputs + 256 * N * 4
    # and at the benchmark shape (40 heads x 75,600 tokens, 100 / 500 clusters)
    s = sv.make_shape(40, 75600, 75600, 128, 100, 500, 10, sv.BF16)
    assert sv.workspace_bytes(s) <= 3 * 2 ** 30


def test_probe_noalloc_validation():
    """svgear_probe_noalloc validates like svgear_probe, and rejects a shape whose
    probe scratch exceeds its 64 MiB device array, before any device call."""
    L = sv.load()
    s = _shape()
    r = ctypes.byref
    assert L.svgear_probe_noalloc(r(s), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None) \
        == sv.E_NULL
    assert L.svgear_probe_noalloc(r(s), FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None) \
        == sv.E_ALIGN
    for flags in (sv.LABELS_GIVEN, sv.PROBE_SCORE | sv.PROBE_LOGIT, 32):
        assert L.svgear_probe_noalloc(r(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, flags, FAKE, FAKE,
                                      None) == sv.E_ARG
    assert L.svgear_probe_noalloc(r(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, sv.DEBUG_EPS, FAKE, None,
                                  None) == sv.E_NULL
    big = sv.make_shape(40, 75600, 75600, 128, 1000, 1000, 10, sv.BF16)   # 160 MB of sbar alone
    assert L.svgear_probe_noalloc(r(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None) \
        == sv.E_WORKSPACE
    bad = _shape(d=32)
    assert L.svgear_probe_noalloc(r(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None) \
        == sv.E_SHAPE
