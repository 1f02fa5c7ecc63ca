"""GPU parity of the routing variants, end to end on one clustering: the
logit-only probe, the attention-score comparator, and per-query-cluster
budgets (with the value-aware and the score ratio).  The library clusters once
(svgear_forward), then the variant's probe, route and attention run through
the per-stage entry points; the oracle does the same steps in fp64.

Bars: ratios as in the probe tests (the score ratio to 1e-4 in ln r); the mask
exact except blocks near the selection threshold (1e-5 relative; 3e-3 for the
logit-only ratio and 1e-4 for the score ratio, as wide as their ratio bars); selected cost within the budget;
output within the dtype's tolerance on every sampled row (against the oracle
run with the library's mask on query clusters where a near-threshold block
flipped)."""
import numpy as np
import pytest

import oracle
from sparse_attention_video_flash_amd import svgear as sv
from sparse_attention_video_flash_amd.inputs import WORKLOADS

from gpu_common import RAGGED, check_output, log, near_threshold_ok, reference_rows, shape_of, torch_gpu, upload

pytestmark = pytest.mark.gpu

CASES = {"ragged": (RAGGED, None, 1), "small": (WORKLOADS["small"], None, 7),
         "stress": (WORKLOADS["stress"], [0, 8], 29)}
FLAGS = {"error": 0, "logit": sv.PROBE_LOGIT, "score": sv.PROBE_SCORE}
TOL_THR = {"error": 1e-5, "logit": 3e-3, "score": 1e-4}
VARIANTS = [("logit", False), ("score", False), ("error", True), ("score", True)]
_CLUSTER: dict = {}


def _oracle_clustering(w, host, hi):
    key = (w.name, hi)
    if key not in _CLUSTER:
        q, k, v, iq, ik = (a[hi] for a in host)
        lq, qbar, cq = oracle.kmeans(q, w.Cq, iq, w.iters)
        lk, kbar, ck = oracle.kmeans(k, w.Ck, ik, w.iters)
        _CLUSTER[key] = (lq, qbar, cq, lk, kbar, ck, oracle.group_means(v, lk, w.Ck))
    return _CLUSTER[key]


def _gpu_variant(w, data, rho, mode, per_row):
    torch = torch_gpu()
    H = len(data["heads"])
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    im = sv.alloc_intermediates(shape)
    O = torch.empty_like(data["Q"])
    sv.forward(shape, rho, data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O, ws, im)
    sv.probe(shape, im["qbar"], im["counts_q"], im["Kp"], im["Vp"], im["kbar"], im["vbar"], im["counts_k"],
             im["offsets_k"], im["log_ratio"], ws, flags=FLAGS[mode])
    (sv.route_rows if per_row else sv.route)(shape, rho, im["log_ratio"], im["counts_q"], im["counts_k"],
                                            im["mask"], im["sel_cost"], ws)
    sv.attention(shape, im["Qp"], im["offsets_q"], im["perm_q"], im["Kp"], im["Vp"], im["kbar"], im["vbar"],
                 im["counts_k"], im["offsets_k"], im["mask"], O, ws)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in im.items() if k in ("labels_q", "labels_k", "log_ratio", "mask",
                                                                "sel_cost", "qbar", "kbar")}
    out["O"] = O.float().cpu().numpy()
    return out


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("mode,per_row", VARIANTS)
def test_variant_matches_oracle(case, mode, per_row):
    w, heads, stride = CASES[case]
    data = upload(w, heads)
    q, k, v, iq, ik = data["host"]
    for rho in sorted(set(w.rhos[:1] + (0.3,))):
        log("variant %s per_row=%s %s rho=%g" % (mode, per_row, case, rho))
        got = _gpu_variant(w, data, rho, mode, per_row)
        for hi in range(len(data["heads"])):
            lq, qbar, cq, lk, kbar, ck, vbar = _oracle_clustering(w, data["host"], hi)
            np.testing.assert_array_equal(got["labels_q"][hi], lq)
            np.testing.assert_array_equal(got["labels_k"][hi], lk)
            if mode == "score":
                lr = oracle.score_log(qbar, cq, kbar, ck)
                # ratio from the fp32 centroids the library holds
                lr32 = oracle.score_log(got["qbar"][hi], cq, got["kbar"][hi], ck)
                fin = np.isfinite(lr32)
                assert (np.isfinite(got["log_ratio"][hi]) == fin).all()
                dev = np.abs(got["log_ratio"][hi][fin] - lr32[fin])
                assert (dev <= 1e-4 + 1e-6 * np.abs(lr32[fin])).all(), float(dev.max())
            else:
                lr = oracle.probe_log(qbar, cq, k[hi], v[hi], lk, kbar, vbar, ck, logit_only=mode == "logit")
            if per_row:
                mask, used = oracle.route_rows(lr, cq, ck, rho, w.N)
                nd = sum(near_threshold_ok(got["mask"][hi][c:c + 1], mask[c:c + 1], lr[c:c + 1], TOL_THR[mode])
                         for c in range(w.Cq))
                for c in range(w.Cq):
                    cost = int((got["mask"][hi][c].astype(np.int64) * ck).sum()) * int(cq[c])
                    assert cost <= oracle.budget(rho, int(cq[c]), w.N)
            else:
                mask, used = oracle.route(lr, cq, ck, rho, w.N, w.N)
                nd = near_threshold_ok(got["mask"][hi], mask, lr, tol=TOL_THR[mode])
                assert int(got["sel_cost"][hi]) <= oracle.budget(rho, w.N, w.N)
            if nd == 0:
                assert int(got["sel_cost"][hi]) == used
            rows = np.arange(0, w.N, stride)
            ref, nflip = reference_rows(q[hi], k[hi], v[hi], lq, lk, kbar, vbar, ck, mask, got["mask"][hi], rows)
            check_output(got["O"][hi][rows], ref, w.dtype,
                         "%s head %d rho=%g (%d rows on flipped clusters)" % (case, hi, rho, nflip))
            log("  head %d: %d near-threshold mask differences" % (hi, nd))
