"""Shared helpers of the GPU parity tests: device upload of seeded inputs, one
library forward with every intermediate kept, and oracle references."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from sparse_attention_video_flash_amd import svgear as sv
from sparse_attention_video_flash_amd.inputs import WORKLOADS, Mixture, Workload, generate_head

# A shape that spans several tiles and leaves ragged tails everywhere:
# 1380 tokens (not a multiple of 32, 64 or 256), odd cluster counts.
RAGGED = Workload("ragged", 3, (3, 20, 23), 128, "bf16", 13, 37, 10, (0.3,), 5,
                  (Mixture((0, 3), 24, (2, 3, 4), 0.25, "normal", 0.08, 2.0, "add"),))

TOL = {"fp32": dict(rel_l2=1e-5, max_abs=1e-4), "bf16": dict(rel_l2=5e-3, max_abs=2e-2)}


def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    sv.load()  # a GPU run must have the library: raises if it is missing
    return torch


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(w: Workload, heads=None):
    """Seeded inputs of ``heads`` as device tensors (+ the host float32 copies)."""
    torch = torch_gpu()
    heads = list(range(w.H)) if heads is None else list(heads)
    parts = [generate_head(w, h) for h in heads]
    q, k, v, iq, ik = (np.stack([p[i] for p in parts]) for i in range(5))
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)  # noqa: E731
    return dict(Q=dev(q, et), K=dev(k, et), V=dev(v, et), init_q=dev(iq, torch.int32),
                init_k=dev(ik, torch.int32), host=(q, k, v, iq, ik), heads=heads)


def shape_of(w: Workload, H: int, iters=None):
    return sv.make_shape(H, w.N, w.N, w.d, w.Cq, w.Ck, w.iters if iters is None else iters,
                         sv.BF16 if w.dtype == "bf16" else sv.F32)


def gpu_forward(w: Workload, rho: float, data=None, heads=None):
    """One svgear_forward call with every intermediate in its own tensor."""
    torch = torch_gpu()
    data = data or upload(w, heads)
    H = len(data["heads"])
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    im = sv.alloc_intermediates(shape)
    O = torch.empty_like(data["Q"])
    sv.forward(shape, rho, data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O, ws, im)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in im.items()}
    out["O"] = O.float().cpu().numpy()
    return out, data


def oracle_head(w: Workload, data, hi: int, rho: float, rows=None, want_eps=False):
    q, k, v, iq, ik = (a[hi] for a in data["host"])
    return oracle.forward_head(q, k, v, iq, ik, w.Cq, w.Ck, rho, iters=w.iters, rows=rows, want_eps=want_eps)


def group_lse(L, labels, C: int):
    """log-sum-exp of the columns of L [R, N] grouped by ``labels`` [N] -> [R, C]."""
    L = np.asarray(L, np.float64)
    M = np.full((L.shape[0], C), -np.inf)
    np.maximum.at(M.T, labels, L.T)
    S = np.zeros_like(M)
    with np.errstate(invalid="ignore"):
        np.add.at(S.T, labels, np.exp(L.T - M.T[labels]))
    with np.errstate(divide="ignore"):
        return np.where(np.isfinite(M), M + np.log(S), -np.inf)


def probe_log_floors(qbar, kbar, vbar, K, V, labels_k, counts_k):
    """ln of the comparison floors of the probe, 1e-4 times the scale of the two
    terms whose difference is e:  per key  a^2 ||vbar||^2 + b^2 ||v_j||^2,  per
    block the mean of that over the block's keys (a = e^{tau qbar.kbar},
    b = e^{tau qbar.k_j}), all in the log domain."""
    qbar, kbar, vbar, K, V = (np.asarray(x, np.float64) for x in (qbar, kbar, vbar, K, V))
    tau = 1.0 / np.sqrt(qbar.shape[1])
    C = kbar.shape[0]
    with np.errstate(divide="ignore"):
        la2 = 2 * tau * qbar @ kbar.T + np.log((vbar ** 2).sum(1))[None, :]    # [Cq, Ck]
        lb2 = 2 * tau * qbar @ K.T + np.log((V ** 2).sum(1))[None, :]          # [Cq, Nk]
        lmean = group_lse(lb2, labels_k, C) - np.log(np.maximum(counts_k, 1))[None, :]
    f = np.log(1e-4)
    return f + np.logaddexp(la2, lmean), f + np.logaddexp(la2[:, labels_k], lb2)


def log_close(l_gpu, l_ref, l_floor, rtol=1e-3):
    """|x_gpu - x_ref| <= rtol * max(x_ref, floor) for x = exp(l), evaluated in the
    log domain; -inf (an exact zero) must be matched by -inf.  Returns (bad, dev)."""
    l_gpu = np.asarray(l_gpu, np.float64)
    l_ref = np.asarray(l_ref, np.float64)
    lf = np.maximum(l_ref, l_floor)
    with np.errstate(over="ignore", invalid="ignore"):
        dev = np.abs(np.exp(l_gpu - lf) - np.exp(l_ref - lf))
    both_zero = (l_ref == -np.inf) & (l_gpu == -np.inf)
    bad = ~(both_zero | (dev <= rtol))
    return bad, np.where(both_zero, 0.0, dev)


def near_threshold_ok(mask_gpu, mask_ref, log_ratio, tol=1e-5):
    """Mask mismatches are allowed only for blocks within ``tol`` relative of the
    oracle's selection threshold (the ratio of the first unselected block):
    |ln r - ln r_thr| <= tol.  Returns the number of mismatches (asserts)."""
    diff = mask_gpu != mask_ref
    if not diff.any():
        return 0
    flat = np.asarray(log_ratio, np.float64).reshape(-1)
    order = np.lexsort((np.arange(flat.size), -flat))
    nsel = int(mask_ref.sum())
    assert nsel < flat.size, "mask differs although every block is selected"
    thr = flat[order[nsel]]
    with np.errstate(invalid="ignore"):
        near = (log_ratio == thr) | (np.abs(log_ratio - thr) <= tol)
    assert (~diff | near).all(), ("mask mismatch away from the threshold", int(diff.sum()))
    return int(diff.sum())


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_output(got, ref, dtype: str, what=""):
    """Output bar: rel-L2 and max-abs.  The max-abs bar was derived for outputs
    of magnitude at most 4 (bf16 storage rounds to half an ulp, 2^-9 relative);
    for larger outputs it scales with the largest reference magnitude / 4."""
    t = TOL[dtype]
    r = rel_l2(got, ref)
    m = float(np.abs(np.asarray(got, np.float64) - ref).max()) if np.size(ref) else 0.0
    big = float(np.abs(ref).max()) if np.size(ref) else 0.0
    tol_abs = t["max_abs"] * max(1.0, big / 4.0)
    log("  %s rel_l2=%.3e max_abs=%.3e (tol %.0e / %.1e, max |o| %.3g)"
        % (what, r, m, t["rel_l2"], tol_abs, big))
    assert r <= t["rel_l2"], (what, r)
    assert m <= tol_abs, (what, m)


def reference_rows(q, k, v, lq, lk, kbar, vbar, ck, mask_ref, mask_gpu, rows):
    """Oracle output on ``rows``: with the oracle's mask where the row's query
    cluster routes as the oracle does, and with the library's mask (already
    vetted by near_threshold_ok) on the clusters where a near-threshold block
    flipped, so that every sampled row is compared."""
    same = (mask_gpu == mask_ref).all(axis=1)[lq[rows]]
    ref = np.empty((len(rows), q.shape[1]), np.float64)
    if same.any():
        ref[same] = oracle.hybrid(q, k, v, lq, lk, kbar, vbar, ck, mask_ref, rows[same])
    if (~same).any():
        ref[~same] = oracle.hybrid(q, k, v, lq, lk, kbar, vbar, ck, mask_gpu, rows[~same])
    return ref, int((~same).sum())


__all__ = ["RAGGED", "WORKLOADS", "torch_gpu", "upload", "shape_of", "gpu_forward", "oracle_head", "rel_l2",
           "check_output", "log", "TOL", "group_lse", "probe_log_floors", "log_close", "near_threshold_ok",
           "reference_rows"]
