"""fp64 CPU oracle for one SVG-EAR routed attention call (ctypes wrapper).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` import this module.
It shares no code with the HIP library: it loads its own C library,
``oracle/libsvgear_oracle.so``, built from ``oracle/svgear_oracle.c`` with gcc
(``build()``; also built on first use when missing or older than the source).

The arithmetic lives in the C file; this module only marshals numpy arrays.
``forward_head`` composes the five steps of the pipeline paragraph of the
SVG-EAR review page (cluster and reorder, probe, ratio, greedy route, hybrid
output) for one head.  Parity status of each step:
k-means, permutation, means, route and the hybrid output are pinned by tests
against library routines, closed forms and brute force; the probe on generic data
is pinned only through its special cases and a brute-force block sum.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svgear_oracle.c")
_LIB = os.path.join(_HERE, "libsvgear_oracle.so")
_lock = threading.Lock()
_lib = None

_I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_U8P = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, -O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _ptr_or_null(t):
    class _P:
        @classmethod
        def from_param(cls, obj):
            if obj is None:
                return None
            return t.from_param(obj)
    return _P


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = ctypes.CDLL(_LIB)
            i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
            L.svgo_assign.argtypes = [i32, i32, i32, _F64P, _F64P, _I32P]
            L.svgo_update.argtypes = [i32, i32, i32, _F64P, _I32P, _F64P, _I32P]
            L.svgo_kmeans.argtypes = [i32, i32, i32, _F64P, _I32P, i32, _I32P, _F64P, _I32P]
            L.svgo_permutation.argtypes = [i32, i32, _I32P, _I32P, _I32P, _I32P, _I32P]
            L.svgo_group_means.argtypes = [i32, i32, i32, _F64P, _I32P, _F64P]
            L.svgo_probe.argtypes = [i32, i32, i32, i32, _F64P, _I32P, _F64P, _F64P, _I32P, _F64P,
                                     _F64P, _I32P, _ptr_or_null(_F64P), _F64P]
            L.svgo_probe_log.argtypes = [i32, i32, i32, i32, _F64P, _I32P, _F64P, _F64P, _I32P, _F64P,
                                         _F64P, _I32P, _ptr_or_null(_F64P), _F64P, i32]
            L.svgo_score_log.argtypes = [i32, i32, i32, _F64P, _I32P, _F64P, _I32P, _F64P]
            L.svgo_route_optimal.argtypes = [i32, i32, _F64P, _I32P, _I32P, i64, _U8P,
                                             ctypes.POINTER(ctypes.c_double)]
            L.svgo_route_optimal.restype = i64
            L.svgo_budget.argtypes = [f64, i32, i32]
            L.svgo_budget.restype = i64
            L.svgo_route.argtypes = [i32, i32, _F64P, _I32P, _I32P, i64, _U8P]
            L.svgo_route.restype = i64
            L.svgo_hybrid.argtypes = [i32, i32, i32, i32, i32, _F64P, _F64P, _F64P, _I32P, _I32P,
                                      _F64P, _F64P, _I32P, _U8P, i32, _ptr_or_null(_I32P), _F64P]
            L.svgo_num_threads.argtypes = []
            _lib = L
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)


def num_threads() -> int:
    return int(lib().svgo_num_threads())


def assign(X, cent):
    X, cent = _f64(X), _f64(cent)
    labels = np.empty(X.shape[0], np.int32)
    _check(lib().svgo_assign(X.shape[0], X.shape[1], cent.shape[0], X, cent, labels))
    return labels


def update(X, labels, cent_prev):
    X = _f64(X)
    cent = _f64(cent_prev).copy()
    counts = np.empty(cent.shape[0], np.int32)
    _check(lib().svgo_update(X.shape[0], X.shape[1], cent.shape[0], X, _i32(labels), cent, counts))
    return cent, counts


def kmeans(X, C: int, init, iters: int = 10):
    """Lloyd's k-means from token indices ``init``: (labels, centroids, counts)."""
    X = _f64(X)
    N, d = X.shape
    labels = np.empty(N, np.int32)
    cent = np.empty((C, d), np.float64)
    counts = np.empty(C, np.int32)
    _check(lib().svgo_kmeans(N, d, C, X, _i32(init), iters, labels, cent, counts))
    return labels, cent, counts


def permutation(labels, C: int):
    """Stable counting sort: (counts, offsets[C+1], perm, inv_perm)."""
    labels = _i32(labels)
    N = labels.shape[0]
    counts = np.empty(C, np.int32)
    offsets = np.empty(C + 1, np.int32)
    perm = np.empty(N, np.int32)
    inv = np.empty(N, np.int32)
    _check(lib().svgo_permutation(N, C, labels, counts, offsets, perm, inv))
    return counts, offsets, perm, inv


def group_means(Y, labels, C: int):
    Y = _f64(Y)
    out = np.empty((C, Y.shape[1]), np.float64)
    _check(lib().svgo_group_means(Y.shape[0], Y.shape[1], C, Y, _i32(labels), out))
    return out


def probe(qbar, counts_q, K, V, labels_k, kbar, vbar, counts_k, want_eps: bool = False):
    """Block ratios r[Cq, Ck] (and e[Cq, Nk] in key token order if ``want_eps``)."""
    qbar, K, V, kbar, vbar = _f64(qbar), _f64(K), _f64(V), _f64(kbar), _f64(vbar)
    Cq, d = qbar.shape
    Nk = K.shape[0]
    Ck = kbar.shape[0]
    ratio = np.empty((Cq, Ck), np.float64)
    eps = np.empty((Cq, Nk), np.float64) if want_eps else None
    _check(lib().svgo_probe(Cq, Nk, Ck, d, qbar, _i32(counts_q), K, V, _i32(labels_k), kbar, vbar,
                            _i32(counts_k), eps, ratio))
    return (ratio, eps) if want_eps else ratio


def probe_log(qbar, counts_q, K, V, labels_k, kbar, vbar, counts_k, want_eps: bool = False,
              logit_only: bool = False):
    """ln r[Cq, Ck] (and ln e[Cq, Nk] in key token order if ``want_eps``), the
    larger exponential factored out so nothing overflows; -inf where r = 0.
    ``logit_only``: the estimate without values, (e^{tau qbar.kbar} - e^{tau qbar.k})^2."""
    qbar, K, V, kbar, vbar = _f64(qbar), _f64(K), _f64(V), _f64(kbar), _f64(vbar)
    Cq, d = qbar.shape
    Nk = K.shape[0]
    Ck = kbar.shape[0]
    lr = np.empty((Cq, Ck), np.float64)
    le = np.empty((Cq, Nk), np.float64) if want_eps else None
    _check(lib().svgo_probe_log(Cq, Nk, Ck, d, qbar, _i32(counts_q), K, V, _i32(labels_k), kbar, vbar,
                                _i32(counts_k), le, lr, 1 if logit_only else 0))
    return (lr, le) if want_eps else lr


def score_log(qbar, counts_q, kbar, counts_k):
    """Attention-score comparator, ln r[Cq, Ck]: the centroid-estimated attention
    mass of block (c, g) per pair of the block, -inf where the block is empty."""
    qbar, kbar = _f64(qbar), _f64(kbar)
    Cq, d = qbar.shape
    Ck = kbar.shape[0]
    lr = np.empty((Cq, Ck), np.float64)
    _check(lib().svgo_score_log(Cq, Ck, d, qbar, _i32(counts_q), kbar, _i32(counts_k), lr))
    return lr


def budget(rho: float, Nq: int, Nk: int) -> int:
    return int(lib().svgo_budget(float(rho), int(Nq), int(Nk)))


def route(ratio, counts_q, counts_k, rho: Optional[float] = None, Nq: Optional[int] = None,
          Nk: Optional[int] = None, budget_pairs: Optional[int] = None):
    """Greedy selection: (mask[Cq, Ck] uint8, selected cost)."""
    ratio = _f64(ratio)
    Cq, Ck = ratio.shape
    if budget_pairs is None:
        budget_pairs = budget(rho, Nq, Nk)
    mask = np.empty((Cq, Ck), np.uint8)
    used = lib().svgo_route(Cq, Ck, ratio, _i32(counts_q), _i32(counts_k), int(budget_pairs), mask)
    if used < 0:
        raise ValueError("oracle route rejected its arguments (code %d)" % used)
    return mask, int(used)


def route_optimal(log_ratio, counts_q, counts_k, budget_pairs: int):
    """Exact 0-1 knapsack selection (dynamic programming over integer costs):
    (mask, selected cost, value) with value = sum over selected blocks of
    cost * e^{ln r - max ln r}; greedy's value on the same scale is
    ``knapsack_value(mask, ...)``."""
    lr = _f64(log_ratio)
    Cq, Ck = lr.shape
    mask = np.empty((Cq, Ck), np.uint8)
    val = ctypes.c_double(0.0)
    used = lib().svgo_route_optimal(Cq, Ck, lr, _i32(counts_q), _i32(counts_k), int(budget_pairs), mask,
                                    ctypes.byref(val))
    if used < 0:
        raise ValueError("oracle knapsack rejected its arguments (code %d)" % used)
    return mask, int(used), float(val.value)


def knapsack_value(mask, log_ratio, counts_q, counts_k) -> float:
    """sum over selected blocks of cost * e^{ln r - max finite ln r}."""
    lr = np.asarray(log_ratio, np.float64)
    shift = lr[np.isfinite(lr)].max() if np.isfinite(lr).any() else 0.0
    cost = np.outer(np.asarray(counts_q, np.float64), np.asarray(counts_k, np.float64))
    with np.errstate(under="ignore"):
        v = np.where(np.isfinite(lr), cost * np.exp(lr - shift), 0.0)
    return float(v[np.asarray(mask, bool)].sum())


def route_rows(ratio, counts_q, counts_k, rho: float, Nk: int):
    """Per-query-cluster budgets (the review page's future-work reading of the
    density budget: one budget per query cluster).  Row c is routed on its own
    with the greedy rule of ``route`` and the budget floor((rho * n_c) * Nk),
    i.e. the head budget formula with the row's query count.  Returns
    (mask[Cq, Ck] uint8, total selected cost over the rows)."""
    ratio = _f64(ratio)
    Cq, Ck = ratio.shape
    cq = _i32(counts_q)
    mask = np.empty((Cq, Ck), np.uint8)
    total = 0
    for c in range(Cq):
        m, used = route(ratio[c:c + 1], cq[c:c + 1], counts_k, budget_pairs=budget(rho, int(cq[c]), Nk))
        mask[c] = m[0]
        total += used
    return mask, total


def hybrid(Q, K, V, labels_q, labels_k, kbar, vbar, counts_k, mask, rows=None):
    """Hybrid attention output for query tokens ``rows`` (default: all), token order."""
    Q, K, V, kbar, vbar = _f64(Q), _f64(K), _f64(V), _f64(kbar), _f64(vbar)
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    Nq, d = Q.shape
    Nk = K.shape[0]
    Cq, Ck = mask.shape
    rows_a = None if rows is None else _i32(rows)
    nrows = Nq if rows is None else rows_a.shape[0]
    O = np.empty((nrows, d), np.float64)
    _check(lib().svgo_hybrid(Nq, Nk, d, Cq, Ck, Q, K, V, _i32(labels_q), _i32(labels_k), kbar, vbar,
                             _i32(counts_k), mask, nrows, rows_a, O))
    return O


def forward_head(Q, K, V, init_q, init_k, Cq: int, Ck: int, rho: float, iters: int = 10,
                 rows: Optional[Sequence[int]] = None, want_eps: bool = False, ratio_mode: str = "error",
                 per_row: bool = False) -> Dict[str, np.ndarray]:
    """All five steps for one head; returns every intermediate and the output.
    ``ratio_mode``: "error" (the value-aware probe), "logit" (its logit-only
    variant) or "score" (the attention-score comparator); ``per_row`` routes
    with one budget per query cluster instead of one per head."""
    if ratio_mode not in ("error", "logit", "score"):
        raise ValueError("ratio_mode must be error, logit or score")
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    Nq, Nk = Q.shape[0], K.shape[0]
    lq, qbar, cq = kmeans(Q, Cq, init_q, iters)
    lk, kbar, ck = kmeans(K, Ck, init_k, iters)
    cq2, offq, permq, invq = permutation(lq, Cq)
    ck2, offk, permk, invk = permutation(lk, Ck)
    vbar = group_means(V, lk, Ck)
    if ratio_mode == "score":
        log_ratio, log_eps = score_log(qbar, cq, kbar, ck), None
        want_eps = False
    else:
        pr = probe_log(qbar, cq, K, V, lk, kbar, vbar, ck, want_eps=want_eps, logit_only=ratio_mode == "logit")
        log_ratio, log_eps = pr if want_eps else (pr, None)
    # ln is increasing, so routing on ln r visits blocks in the order of r
    if per_row:
        mask, used = route_rows(log_ratio, cq, ck, rho, Nk)
    else:
        mask, used = route(log_ratio, cq, ck, rho, Nq, Nk)
    O = hybrid(Q, K, V, lq, lk, kbar, vbar, ck, mask, rows)
    with np.errstate(over="ignore"):
        ratio = np.exp(log_ratio)
    out = dict(labels_q=lq, qbar=qbar, counts_q=cq, offsets_q=offq, perm_q=permq, inv_perm_q=invq,
               labels_k=lk, kbar=kbar, counts_k=ck, offsets_k=offk, perm_k=permk, inv_perm_k=invk,
               vbar=vbar, log_ratio=log_ratio, ratio=ratio, mask=mask, sel_cost=np.int64(used),
               budget=np.int64(budget(rho, Nq, Nk)), O=O)
    if want_eps:
        out["log_eps2"] = log_eps
        with np.errstate(over="ignore"):
            out["eps2"] = np.exp(log_eps)
    return out
