"""Pins of the oracle's hybrid output (step 4 of the SVG-EAR review page's
pipeline paragraph; centroid compensation of skipped blocks, German summary 2A)
against dense attention, closed forms and invariances.  CPU only."""
import numpy as np
import pytest

import oracle
from sparse_attention_video_flash_amd.inputs import WORKLOADS, Mixture, Workload, generate_head


def _dense(Q, K, V):
    s = (Q @ K.T) / np.sqrt(Q.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=1, keepdims=True)) @ V


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_full_density_is_dense_attention():
    w = WORKLOADS["tiny"]
    q, k, v, iq, ik = generate_head(w, 0)
    r = oracle.forward_head(q, k, v, iq, ik, w.Cq, w.Ck, 1.0)
    assert r["mask"].all()
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    assert _rel(r["O"], _dense(Q, K, V)) <= 1e-12


def test_low_density_differs_from_dense():
    """Guard against a path that silently computes dense attention."""
    w = WORKLOADS["tiny"]
    q, k, v, iq, ik = generate_head(w, 0)
    r = oracle.forward_head(q, k, v, iq, ik, w.Cq, w.Ck, 0.25)
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    assert 1e-3 < _rel(r["O"], _dense(Q, K, V)) < 0.5
    assert 0 < r["mask"].sum() < r["mask"].size


@pytest.mark.parametrize("rho", [0.0, 0.1, 0.3])
def test_singleton_key_clusters_compensate_exactly(rho):
    """Ck = Nk: each skipped key is replaced by itself, so every density gives dense attention."""
    w = WORKLOADS["tiny"]
    q, k, v, iq, _ = generate_head(w, 0)
    q, k, v = q[:200], k[:96], v[:96]
    r = oracle.forward_head(q, k, v, np.arange(8, dtype=np.int32) * 20, np.arange(96, dtype=np.int32),
                            8, 96, rho, iters=3)
    np.testing.assert_array_equal(r["labels_k"], np.arange(96))
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    assert _rel(r["O"], _dense(Q, K, V)) <= 1e-12


@pytest.mark.parametrize("rho", [0.0, 0.2, 0.5])
def test_keys_identical_within_clusters_compensate_exactly(rho):
    """k_j = kbar_g for every key: m_g * exp(q.kbar_g) * vbar_g equals the exact
    sum over the cluster, whatever V is."""
    rng = np.random.default_rng(9)
    G, per, d = 7, 9, 32
    kc = rng.standard_normal((G, d))
    lab = np.repeat(np.arange(G), per)
    rng.shuffle(lab)
    lab[lab == 6] = 5               # uneven cluster sizes; cluster 6 keeps one member below
    lab[0] = 6
    K = kc[lab]
    V = rng.standard_normal((K.shape[0], d))
    Q = rng.standard_normal((50, d))
    init_k = np.array([np.flatnonzero(lab == g)[0] for g in range(G)], np.int32)
    r = oracle.forward_head(Q, K, V, np.arange(4, dtype=np.int32), init_k, 4, G, rho, iters=3)
    np.testing.assert_array_equal(r["labels_k"], lab)
    assert _rel(r["O"], _dense(Q, K, V)) <= 1e-12


def test_zero_density_single_key_cluster_gives_mean_of_values():
    w = WORKLOADS["tiny"]
    q, k, v, iq, _ = generate_head(w, 0)
    r = oracle.forward_head(q, k, v, iq, np.array([3], np.int32), w.Cq, 1, 0.0, iters=2)
    assert r["mask"].sum() == 0
    np.testing.assert_allclose(r["O"], np.broadcast_to(v.astype(np.float64).mean(0), r["O"].shape),
                               rtol=0, atol=1e-13)


def _blocked_output(Q, K, V, r):
    """Second formulation: walk query clusters and key clusters in the reordered
    (cluster-contiguous) layout, block by block, then undo the reordering."""
    tau = 1.0 / np.sqrt(Q.shape[1])
    Qp, Kp, Vp = Q[r["perm_q"]], K[r["perm_k"]], V[r["perm_k"]]
    oq, ok = r["offsets_q"], r["offsets_k"]
    Cq, Ck = r["mask"].shape
    Op = np.zeros_like(Qp)
    for c in range(Cq):
        qs = Qp[oq[c]:oq[c + 1]]
        if qs.shape[0] == 0:
            continue
        logits, vals = [], []
        for g in range(Ck):
            m = ok[g + 1] - ok[g]
            if m == 0:
                continue
            if r["mask"][c, g]:
                logits.append(tau * qs @ Kp[ok[g]:ok[g + 1]].T)
                vals.append(Vp[ok[g]:ok[g + 1]])
            else:
                logits.append(tau * qs @ r["kbar"][g][:, None] + np.log(m))
                vals.append(r["vbar"][g][None, :])
        s = np.concatenate(logits, axis=1)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        Op[oq[c]:oq[c + 1]] = (p @ np.concatenate(vals, axis=0)) / p.sum(axis=1, keepdims=True)
    return Op[r["inv_perm_q"]]


@pytest.mark.parametrize("rho", [0.1, 0.25, 0.6])
def test_blocked_formulation_agrees(rho):
    w = WORKLOADS["tiny"]
    q, k, v, iq, ik = generate_head(w, 0)
    r = oracle.forward_head(q, k, v, iq, ik, w.Cq, w.Ck, rho)
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    assert _rel(r["O"], _blocked_output(Q, K, V, r)) <= 1e-12


def test_output_is_equivariant_under_token_permutation():
    """Relabelling the tokens (initial indices mapped along) permutes the output
    rows the same way: nothing depends on where a token sits in the sequence."""
    w = Workload("perm", 1, (2, 16, 16), 32, "bf16", 6, 12, 10, (0.3,), 21,
                 (Mixture((0, 1), 16, (1, 4, 4), 0.3, "normal", 0.05, 2.0, "add"),))
    q, k, v, iq, ik = generate_head(w, 0)
    rng = np.random.default_rng(0)
    pq = rng.permutation(q.shape[0])
    pk = rng.permutation(k.shape[0])
    inv_pq = np.argsort(pq)
    inv_pk = np.argsort(pk)
    a = oracle.forward_head(q, k, v, iq, ik, 6, 12, 0.3)
    b = oracle.forward_head(q[pq], k[pk], v[pk], inv_pq[iq].astype(np.int32),
                            inv_pk[ik].astype(np.int32), 6, 12, 0.3)
    np.testing.assert_array_equal(b["labels_q"], a["labels_q"][pq])
    np.testing.assert_array_equal(b["labels_k"], a["labels_k"][pk])
    np.testing.assert_array_equal(b["mask"], a["mask"])
    np.testing.assert_allclose(b["O"], a["O"][pq], rtol=0, atol=1e-12)


def test_row_subset_equals_full_rows():
    w = WORKLOADS["tiny"]
    q, k, v, iq, ik = generate_head(w, 0)
    r = oracle.forward_head(q, k, v, iq, ik, w.Cq, w.Ck, 0.25)
    rows = np.arange(3, q.shape[0], 37, dtype=np.int32)
    sub = oracle.hybrid(q, k, v, r["labels_q"], r["labels_k"], r["kbar"], r["vbar"], r["counts_k"],
                        r["mask"], rows)
    np.testing.assert_array_equal(sub, r["O"][rows])
