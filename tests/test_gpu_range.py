"""GPU parity of the clustering over the input range, and device-detected data
errors reported through the C ABI.

The exact centroid sums pick their fixed-point scale per head from the largest
magnitude, so values of several hundred to a few thousand, and heads of only a
few tokens, must still give labels, permutations and centroids bit-identical
to the fp64 oracle (review page, inference-pipeline step 1: the clustering and
centroids).  A head with a non-finite value, or a non-zero value too small to be
captured next to its largest one, and an initial index outside [0, N), are
reported by svgear_forward under SVGEAR_DEBUG_SYNC (SVGEAR_E_RANGE, SVGEAR_E_ARG);
every kernel still runs to its end on such data (labels stay in range)."""
import dataclasses

import numpy as np
import pytest

import oracle
from sparse_attention_video_flash_amd import svgear as sv
from sparse_attention_video_flash_amd.inputs import WORKLOADS, Mixture, Workload, generate_head, round_to_bf16

from gpu_common import RAGGED, check_output, log, shape_of, torch_gpu

pytestmark = pytest.mark.gpu

# (workload, scale of every value): ragged bf16 d=128 shapes (MFMA screen) and
# the tiny fp32 d=64 shape (exact fp64 assignment), scaled to thousands.
WIDE = {"bf16": (RAGGED, 613.0), "fp32": (WORKLOADS["tiny"], 613.0)}
# a few tokens per head, values around 100 (the fixed-point scale of the
# previous library rounded such values at small N)
SMALL_N = {
    "bf16_n64": Workload("n64", 2, (1, 8, 8), 128, "bf16", 4, 4, 10, (0.5,), 11,
                         (Mixture((0, 2), 4, (1, 2, 2), 0.3),)),
    "fp32_n9": Workload("n9", 2, (1, 3, 3), 64, "fp32", 3, 3, 10, (0.5,), 12,
                        (Mixture((0, 2), 1, (1, 1, 1), 0.3),)),
}


def _data(w: Workload, scale: float):
    """Seeded inputs of every head of w, scaled (and re-rounded for bf16)."""
    heads = [generate_head(w, h) for h in range(w.H)]
    out = []
    for i in range(3):
        x = np.stack([hd[i] for hd in heads]) * np.float32(scale)
        out.append(round_to_bf16(x) if w.dtype == "bf16" else x.astype(np.float32))
    return out + [np.stack([hd[3] for hd in heads]), np.stack([hd[4] for hd in heads])]


def _dev(a, dt):
    torch = torch_gpu()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)


def _cluster_and_check(w, q, k, v, iq, ik):
    torch = torch_gpu()
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    H, N = q.shape[0], q.shape[1]
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    for side, Xh, C, init in ((0, q, w.Cq, iq), (1, k, w.Ck, ik)):
        X = _dev(Xh, et)
        out = dict(labels=torch.empty(H, N, dtype=torch.int32, device="cuda"),
                   cent=torch.empty(H, C, w.d, device="cuda"),
                   counts=torch.empty(H, C, dtype=torch.int32, device="cuda"),
                   offsets=torch.empty(H, C + 1, dtype=torch.int32, device="cuda"),
                   perm=torch.empty(H, N, dtype=torch.int32, device="cuda"),
                   inv_perm=torch.empty(H, N, dtype=torch.int32, device="cuda"), Xp=torch.empty_like(X))
        V = None
        if side == 1:
            V = _dev(v, et)
            out["vbar"] = torch.empty(H, C, w.d, device="cuda")
            out["Vp"] = torch.empty_like(V)
        sv.cluster(shape, side, X, _dev(init, torch.int32), out, ws, V=V, flags=sv.DEBUG_SYNC)
        for hi in range(H):
            lab, cent, counts = oracle.kmeans(Xh[hi], C, init[hi], iters=w.iters)
            c2, offsets, perm, inv = oracle.permutation(lab, C)
            np.testing.assert_array_equal(out["labels"][hi].cpu().numpy(), lab)
            np.testing.assert_array_equal(out["counts"][hi].cpu().numpy(), counts)
            np.testing.assert_array_equal(out["offsets"][hi].cpu().numpy(), offsets)
            np.testing.assert_array_equal(out["perm"][hi].cpu().numpy(), perm)
            np.testing.assert_array_equal(out["inv_perm"][hi].cpu().numpy(), inv)
            np.testing.assert_array_equal(out["Xp"][hi].float().cpu().numpy(), Xh[hi][perm])
            np.testing.assert_array_equal(out["cent"][hi].cpu().numpy(), cent.astype(np.float32))
            if side == 1:
                vbar = oracle.group_means(v[hi], lab, C)
                np.testing.assert_array_equal(out["vbar"][hi].cpu().numpy(), vbar.astype(np.float32))
        log("  side %d: labels, permutation and centroids bit-exact (max |x| %.1f)"
            % (side, float(np.abs(Xh).max())))


@pytest.mark.parametrize("case", sorted(WIDE))
def test_wide_range_clustering_bit_exact(case):
    w, scale = WIDE[case]
    log("wide-range clustering %s (x %g)" % (case, scale))
    q, k, v, iq, ik = _data(w, scale)
    assert np.abs(k).max() > 1000.0
    _cluster_and_check(w, q, k, v, iq, ik)


@pytest.mark.parametrize("case", sorted(SMALL_N))
def test_small_n_clustering_bit_exact(case):
    w = SMALL_N[case]
    log("small-N clustering %s (N=%d)" % (case, w.N))
    q, k, v, iq, ik = _data(w, 100.0)
    _cluster_and_check(w, q, k, v, iq, ik)


def _exact_means(X, labels, C):
    """Means of the rows of X (bf16 values as float32) per label, each the exact
    rational mean rounded once to fp64: the values are scaled by 2^150 to
    integers, summed exactly, and divided as fractions."""
    from fractions import Fraction
    X = np.asarray(X, np.float64)
    out = np.zeros((C, X.shape[1]))
    for m in range(C):
        rows = X[labels == m]
        if len(rows) == 0:
            continue
        for t in range(X.shape[1]):
            tot = sum(int(v * 2.0 ** 150) for v in rows[:, t])
            out[m, t] = float(Fraction(tot, len(rows) * 2 ** 150))
    return out


def test_two_word_sums_through_the_delta_updates():
    """A head whose values span more than one 64-bit word of the fixed-point
    sums (values near 10^-13 next to values in the hundreds) is summed with two
    words: in the first update, in every later update (which adds only the
    tokens that changed cluster), and in the final means.  Its labels and
    permutation equal the oracle's; its centroids are within one fp32 ulp of
    the exact means of the final labels (the oracle's plain fp64 sums round at
    this span, the device's integer sums do not).  The other heads stay on one
    word and are bit-exact."""
    torch = torch_gpu()
    w = RAGGED
    log("two-word heads through the k-means updates")
    q, k, v, iq, ik = _data(w, 613.0)
    # head 0: coordinate 5 of every token near 10^-13, so that its centroid
    # coordinates are of that size too and show any value the sums dropped
    rng = np.random.default_rng(11)
    for X in (q, k):
        X[0, :, 5] = round_to_bf16((3e-13 * rng.standard_normal(X.shape[1])).astype(np.float32))
    et = torch.bfloat16
    H = q.shape[0]
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    for side, Xh, C, init in ((0, q, w.Cq, iq), (1, k, w.Ck, ik)):
        N = Xh.shape[1]
        X = _dev(Xh, et)
        out = dict(labels=torch.empty(H, N, dtype=torch.int32, device="cuda"),
                   cent=torch.empty(H, C, w.d, device="cuda"),
                   counts=torch.empty(H, C, dtype=torch.int32, device="cuda"),
                   offsets=torch.empty(H, C + 1, dtype=torch.int32, device="cuda"),
                   perm=torch.empty(H, N, dtype=torch.int32, device="cuda"),
                   inv_perm=torch.empty(H, N, dtype=torch.int32, device="cuda"), Xp=torch.empty_like(X))
        V = None
        if side == 1:
            V = _dev(v, et)
            out["vbar"] = torch.empty(H, C, w.d, device="cuda")
            out["Vp"] = torch.empty_like(V)
        sv.cluster(shape, side, X, _dev(init, torch.int32), out, ws, V=V, flags=sv.DEBUG_SYNC)
        for hi in range(H):
            lab, cent, counts = oracle.kmeans(Xh[hi], C, init[hi], iters=w.iters)
            np.testing.assert_array_equal(out["labels"][hi].cpu().numpy(), lab)
            np.testing.assert_array_equal(out["counts"][hi].cpu().numpy(), counts)
            perm = oracle.permutation(lab, C)[2]
            np.testing.assert_array_equal(out["perm"][hi].cpu().numpy(), perm)
            np.testing.assert_array_equal(out["Xp"][hi].float().cpu().numpy(), Xh[hi][perm])
            got = out["cent"][hi].cpu().numpy()
            if hi == 0:   # non-empty clusters (an empty one keeps its centroid of an earlier iteration)
                ref = _exact_means(Xh[hi], lab, C).astype(np.float32)
                ulp = np.spacing(np.abs(ref))
                ne = counts > 0
                assert ne.sum() > C // 2
                assert (np.abs(got - ref)[ne] <= ulp[ne]).all(), float((np.abs(got - ref) / ulp)[ne].max())
            else:
                np.testing.assert_array_equal(got, cent.astype(np.float32))
        log("  side %d: labels and permutation exact, two-word head within one ulp" % side)


def test_many_tied_centroids_take_the_blocked_recheck():
    """Seventy initial centroids on one token: every token near it has more
    than RC_MAXCAND = 64 exactly tied candidates, so its exact settlement takes
    the block-by-block candidate path; labels (lowest index on ties), counts,
    permutation and centroids stay bit-exact with the oracle."""
    w = Workload("ties", 2, (3, 20, 23), 128, "bf16", 16, 100, 6, (0.3,), 21,
                 (Mixture((0, 2), 24, (2, 3, 4), 0.25, "normal", 0.08, 2.0, "add"),))
    log("clustering with 70 coincident initial centroids")
    q, k, v, iq, ik = _data(w, 1.0)
    ik = ik.copy()
    ik[:, :70] = ik[:, :1]
    _cluster_and_check(w, q, k, v, iq, ik)


def test_wide_range_forward_matches_oracle():
    """End to end at values in the thousands (logits in the millions: the
    softmax picks single keys); the output bar scales with the output."""
    torch = torch_gpu()
    w, scale = WIDE["bf16"]
    q, k, v, iq, ik = _data(w, scale)
    rho = w.rhos[0]
    H = q.shape[0]
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    O = torch.empty(H, w.N, w.d, dtype=torch.bfloat16, device="cuda")
    im = sv.alloc_intermediates(shape)
    sv.forward(shape, rho, _dev(q, torch.bfloat16), _dev(k, torch.bfloat16), _dev(v, torch.bfloat16),
               _dev(iq, torch.int32), _dev(ik, torch.int32), O, ws, im, flags=sv.DEBUG_SYNC)
    got = O.float().cpu().numpy()
    mask = im["mask"].cpu().numpy()
    for hi in range(H):
        lq, qbar, cq = oracle.kmeans(q[hi], w.Cq, iq[hi], w.iters)
        lk, kbar, ck = oracle.kmeans(k[hi], w.Ck, ik[hi], w.iters)
        vbar = oracle.group_means(v[hi], lk, w.Ck)
        np.testing.assert_array_equal(im["labels_q"][hi].cpu().numpy(), lq)
        np.testing.assert_array_equal(im["labels_k"][hi].cpu().numpy(), lk)
        # output against the oracle evaluated with the library's own routing
        ref = oracle.hybrid(q[hi], k[hi], v[hi], lq, lk, kbar, vbar, ck, mask[hi])
        check_output(got[hi], ref, "bf16", "wide-range head %d" % hi)


def _forward_status(w, q, k, v, iq, ik):
    torch = torch_gpu()
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    H = q.shape[0]
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    O = torch.empty(H, w.N, w.d, dtype=et, device="cuda")
    try:
        sv.forward(shape, w.rhos[0], _dev(q, et), _dev(k, et), _dev(v, et), _dev(iq, torch.int32),
                   _dev(ik, torch.int32), O, ws, flags=sv.DEBUG_SYNC)
    except sv.SvgearError as e:
        return e.code
    return sv.OK


@pytest.mark.parametrize("case", ["bf16", "fp32"])
def test_forward_reports_data_errors(case):
    w = RAGGED if case == "bf16" else WORKLOADS["tiny"]
    q, k, v, iq, ik = _data(w, 1.0)
    log("data errors %s" % case)
    assert _forward_status(w, q, k, v, iq, ik) == sv.OK
    # a non-finite key
    k2 = k.copy()
    k2[0, 5, 3] = np.inf
    assert _forward_status(w, q, k2, v, iq, ik) == sv.E_RANGE
    # a NaN query
    q2 = q.copy()
    q2[-1, 7, 1] = np.nan
    assert _forward_status(w, q2, k, v, iq, ik) == sv.E_RANGE
    # a value of magnitude 2^56
    v2 = v.copy()
    v2[0, 2, 0] = np.float32(2.0 ** 56)
    assert _forward_status(w, q, k, v2, iq, ik) == sv.E_RANGE
    # a non-zero value below the exactness floor next to a large one (all of its
    # mantissa bits set, so it cannot be a multiple of the resolution)
    v3 = v.copy()
    v3[0, 0, 0] = np.float32(300.0)
    v3[0, 1, 0] = np.float32((1 + 127 / 128) * 2.0 ** -100)
    assert _forward_status(w, q, k, v3, iq, ik) == sv.E_RANGE
    # an initial index outside [0, N)
    ik2 = ik.copy()
    ik2[0, 0] = w.N
    assert _forward_status(w, q, k, v, iq, ik2) == sv.E_ARG
    # the error words do not leak into the next call
    assert _forward_status(w, q, k, v, iq, ik) == sv.OK
