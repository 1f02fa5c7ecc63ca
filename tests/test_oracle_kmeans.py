"""Pins of the oracle's clustering and reordering (step 1 of the SVG-EAR pipeline
paragraph on the review page) against a library routine, closed forms and
invariants.  CPU only."""
import warnings

import numpy as np
import pytest
from scipy.cluster.vq import kmeans2

import oracle
from sparse_attention_video_flash_amd.inputs import WORKLOADS, Mixture, Workload, generate_head


def _tiny():
    w = WORKLOADS["tiny"]
    return w, generate_head(w, 0)


def _small_custom(N_grid=(2, 16, 16), d=32, C=12, seed=7):
    w = Workload("t", 1, N_grid, d, "bf16", C, C, 10, (0.3,), seed,
                 (Mixture((0, 1), 16, (1, 4, 4), 0.3, "normal", 0.05, 2.0, "add"),))
    return w, generate_head(w, 0)


@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_kmeans_matches_scipy_kmeans2(which):
    """Lloyd with given initial centroids, fixed iterations, empty clusters kept:
    scipy.cluster.vq.kmeans2(minit='matrix') is the same algorithm in float64."""
    w, (q, k, v, iq, ik) = _tiny()
    X = {"q": q, "k": k, "v": v}[which].astype(np.float64)
    init = iq if which == "q" else ik
    C = len(init)
    labels, cent, counts = oracle.kmeans(X, C, init, iters=10)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        ref_cent, ref_labels = kmeans2(X, X[init].copy(), iter=10, minit="matrix", missing="warn")
    np.testing.assert_array_equal(labels, ref_labels)
    np.testing.assert_allclose(cent, ref_cent, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(counts, np.bincount(labels, minlength=C))


def test_kmeans_matches_scipy_with_outliers_and_empty_clusters():
    w, (q, k, v, iq, ik) = _small_custom()
    X = q.astype(np.float64)
    # Start two centroids on the same token so that one cluster stays empty.
    init = iq.copy()
    init[1] = init[0]
    labels1, cent1, counts1 = oracle.kmeans(X, len(init), init, iters=1)
    assert counts1[1] == 0, "a duplicated start leaves the higher index empty (ties go low)"
    np.testing.assert_array_equal(cent1[1], X[init[1]])  # empty cluster keeps its centroid
    labels, cent, counts = oracle.kmeans(X, len(init), init, iters=10)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        ref_cent, ref_labels = kmeans2(X, X[init].copy(), iter=10, minit="matrix", missing="warn")
    np.testing.assert_array_equal(labels, ref_labels)
    np.testing.assert_allclose(cent, ref_cent, rtol=0, atol=1e-12)


def test_kmeans_single_cluster_is_global_mean():
    _, (q, *_rest) = _tiny()
    X = q.astype(np.float64)
    labels, cent, counts = oracle.kmeans(X, 1, np.array([5], np.int32), iters=3)
    assert (labels == 0).all() and counts[0] == X.shape[0]
    np.testing.assert_allclose(cent[0], X.mean(axis=0), rtol=0, atol=1e-13)


def test_kmeans_separated_blobs_recover_blob_ids():
    rng = np.random.default_rng(3)
    B, per, d = 6, 40, 16
    centers = rng.standard_normal((B, d)) * 50.0
    blob = np.repeat(np.arange(B), per)
    perm = rng.permutation(B * per)
    blob = blob[perm]
    X = centers[blob] + rng.standard_normal((B * per, d)) * 0.1
    init = np.array([np.flatnonzero(blob == b)[0] for b in range(B)], np.int32)
    labels, cent, counts = oracle.kmeans(X, B, init, iters=10)
    np.testing.assert_array_equal(labels, blob)
    np.testing.assert_array_equal(counts, np.full(B, per))


def test_kmeans_every_token_its_own_cluster():
    _, (q, *_rest) = _tiny()
    X = q[:96].astype(np.float64)
    init = np.arange(96, dtype=np.int32)
    labels, cent, counts = oracle.kmeans(X, 96, init, iters=4)
    np.testing.assert_array_equal(labels, np.arange(96))
    np.testing.assert_array_equal(cent, X)
    assert (counts == 1).all()


def test_kmeans_ties_go_to_lowest_index():
    X = np.array([[0.0, 0.0], [2.0, 0.0], [1.0, 0.0], [1.0, 0.0]])
    cent = np.array([[0.0, 0.0], [2.0, 0.0]])
    labels = oracle.assign(X, cent)
    # tokens 2 and 3 sit exactly halfway: both go to cluster 0
    np.testing.assert_array_equal(labels, [0, 1, 0, 0])


def test_lloyd_objective_never_increases_and_centroids_are_member_means():
    w, (q, k, v, iq, ik) = _small_custom(seed=11)
    X = k.astype(np.float64)
    prev = np.inf
    for it in range(1, 11):
        labels, cent, counts = oracle.kmeans(X, len(ik), ik, iters=it)
        J = float(((X - cent[labels]) ** 2).sum())
        assert J <= prev * (1 + 1e-12)
        prev = J
        sums = np.zeros_like(cent)
        np.add.at(sums, labels, X)
        nz = counts > 0
        np.testing.assert_allclose(cent[nz], sums[nz] / counts[nz, None], rtol=1e-14, atol=1e-14)


def test_permutation_is_the_stable_sort_by_label():
    _, (q, k, v, iq, ik) = _tiny()
    labels, _, _ = oracle.kmeans(k.astype(np.float64), len(ik), ik)
    C = len(ik)
    counts, offsets, perm, inv = oracle.permutation(labels, C)
    np.testing.assert_array_equal(perm, np.argsort(labels, kind="stable"))
    np.testing.assert_array_equal(counts, np.bincount(labels, minlength=C))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(labels, minlength=C))]))
    np.testing.assert_array_equal(inv[perm], np.arange(len(labels)))


def test_group_means_match_bincount_and_identical_members():
    rng = np.random.default_rng(5)
    labels = rng.integers(0, 7, size=300).astype(np.int32)
    labels[labels == 4] = 3  # group 4 empty
    Y = rng.standard_normal((300, 9))
    means = oracle.group_means(Y, labels, 7)
    cnt = np.bincount(labels, minlength=7)
    for t in range(9):
        ref = np.bincount(labels, weights=Y[:, t], minlength=7)
        nz = cnt > 0
        np.testing.assert_allclose(means[nz, t], ref[nz] / cnt[nz], rtol=1e-14, atol=1e-15)
    assert (means[4] == 0).all()
    # members identical within a group: the mean is that member (up to the rounding of the sum)
    base = rng.standard_normal((7, 9))
    got = oracle.group_means(base[labels], labels, 7)
    nz = cnt > 0
    np.testing.assert_allclose(got[nz], base[nz], rtol=1e-14, atol=0)


def test_oracle_rejects_bad_arguments():
    X = np.zeros((4, 2))
    with pytest.raises(ValueError):
        oracle.kmeans(X, 5, np.arange(5, dtype=np.int32))  # C > N
    with pytest.raises(ValueError):
        oracle.kmeans(X, 2, np.array([0, 9], np.int32))    # init out of range
    with pytest.raises(ValueError):
        oracle.permutation(np.array([0, 3], np.int32), 2)  # label out of range
