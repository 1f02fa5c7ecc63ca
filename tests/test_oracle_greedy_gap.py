"""How far the greedy route falls from the exact 0-1 knapsack optimum, on the
small seeded workloads (oracle only, fp64).  Per head and density: the greedy
selection's share of the optimal estimated-error value, and the hybrid output
error against dense attention for both selections at the same budget.

Asserted: greedy never beats the optimum, both stay within the budget, and the
optimum's estimated value is what its mask holds.  The figures are printed
(run with -s) and are reported, not asserted: a larger estimated value need
not mean a smaller output error, since the estimate uses the query centroid."""
import numpy as np
import pytest

import oracle
from sparse_attention_video_flash_amd.inputs import WORKLOADS, Mixture, Workload, generate_head

RAGGED = Workload("ragged", 3, (3, 20, 23), 128, "bf16", 13, 37, 10, (0.3,), 5,
                  (Mixture((0, 3), 24, (2, 3, 4), 0.25, "normal", 0.08, 2.0, "add"),))


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("w", [WORKLOADS["tiny"], RAGGED], ids=["tiny", "ragged"])
def test_greedy_gap_against_knapsack_optimum(w):
    for h in range(w.H):
        q, k, v, iq, ik = generate_head(w, h)
        r = oracle.forward_head(q, k, v, iq, ik, w.Cq, w.Ck, 1.0, iters=w.iters)
        lr, cq, ck = r["log_ratio"], r["counts_q"], r["counts_k"]
        dense = oracle.hybrid(q, k, v, r["labels_q"], r["labels_k"], r["kbar"], r["vbar"], ck,
                              np.ones((w.Cq, w.Ck), np.uint8))
        for rho in (0.05, 0.1, 0.2, 0.3, 0.5):
            B = oracle.budget(rho, w.N, w.N)
            gmask, gused = oracle.route(lr, cq, ck, budget_pairs=B)
            omask, oused, oval = oracle.route_optimal(lr, cq, ck, B)
            gval = oracle.knapsack_value(gmask, lr, cq, ck)
            assert gused <= B and oused <= B
            assert oracle.knapsack_value(omask, lr, cq, ck) == pytest.approx(oval, rel=1e-9)
            assert gval <= oval * (1 + 1e-12)
            errs = []
            for m in (gmask, omask):
                O = oracle.hybrid(q, k, v, r["labels_q"], r["labels_k"], r["kbar"], r["vbar"], ck, m)
                errs.append(_rel_l2(O, dense))
            print("%s head %d rho=%.2f: greedy value gap %.2e (cost %d/%d, opt %d); output rel-L2 "
                  "greedy %.4e, optimal %.4e" % (w.name, h, rho, 1.0 - gval / oval if oval > 0 else 0.0, gused,
                                                  B, oused, errs[0], errs[1]))
