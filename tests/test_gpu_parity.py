"""GPU parity: every stage of libsvgear against the fp64 oracle on the same
seeded inputs, stage by stage (oracle results injected as inputs) and end to
end.  Bars: integer outputs bit-exact; ratios within 1e-3 relative; route mask
bit-exact given the same ratios; output rel-L2 <= 1e-5 (fp32) or <= 5e-3 with
max-abs <= 2e-2 (bf16)."""
import numpy as np
import pytest

import oracle
from sparse_attention_video_flash_amd import svgear as sv

from gpu_common import (RAGGED, WORKLOADS, check_output, gpu_forward, log, log_close, near_threshold_ok,
                        oracle_head, probe_log_floors, reference_rows, shape_of, torch_gpu, upload)

pytestmark = pytest.mark.gpu

CASES = {"tiny": WORKLOADS["tiny"], "ragged": RAGGED, "small": WORKLOADS["small"]}


def _dev(a, dt):
    torch = torch_gpu()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)


def _et(w):
    torch = torch_gpu()
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _oracle_all(w, data, rho, want_eps=False):
    return [oracle_head(w, data, hi, rho, want_eps=want_eps) for hi in range(len(data["heads"]))]


# ----------------------------------------------------------------------------- step 1

@pytest.mark.parametrize("case", ["tiny", "ragged", "small"])
def test_cluster_with_oracle_labels_is_bit_exact(case):
    torch = torch_gpu()
    w = CASES[case]
    log("cluster labels-given %s" % case)
    data = upload(w)
    H = len(data["heads"])
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    q, k, v, iq, ik = data["host"]
    for side, X, Xh, C in ((0, data["Q"], q, w.Cq), (1, data["K"], k, w.Ck)):
        labels = []
        for hi in range(H):
            init = (iq if side == 0 else ik)[hi]
            labels.append(oracle.kmeans(Xh[hi], C, init, iters=w.iters)[0])
        labels = np.stack(labels)
        out = dict(labels=_dev(labels, torch.int32), cent=torch.empty(H, C, w.d, device="cuda"),
                   counts=torch.empty(H, C, dtype=torch.int32, device="cuda"),
                   offsets=torch.empty(H, C + 1, dtype=torch.int32, device="cuda"),
                   perm=torch.empty(H, X.shape[1], dtype=torch.int32, device="cuda"),
                   inv_perm=torch.empty(H, X.shape[1], dtype=torch.int32, device="cuda"),
                   Xp=torch.empty_like(X))
        V = None
        if side == 1:
            out["vbar"] = torch.empty(H, C, w.d, device="cuda")
            out["Vp"] = torch.empty_like(data["V"])
            V = data["V"]
        sv.cluster(shape, side, X, None, out, ws, V=V, flags=sv.LABELS_GIVEN | sv.DEBUG_SYNC)
        for hi in range(H):
            counts, offsets, perm, inv = oracle.permutation(labels[hi], C)
            np.testing.assert_array_equal(out["counts"][hi].cpu().numpy(), counts)
            np.testing.assert_array_equal(out["offsets"][hi].cpu().numpy(), offsets)
            np.testing.assert_array_equal(out["perm"][hi].cpu().numpy(), perm)
            np.testing.assert_array_equal(out["inv_perm"][hi].cpu().numpy(), inv)
            np.testing.assert_array_equal(out["Xp"][hi].float().cpu().numpy(), Xh[hi][perm])
            means = oracle.group_means(Xh[hi], labels[hi], C)
            np.testing.assert_array_equal(out["cent"][hi].cpu().numpy(), means.astype(np.float32))
            if side == 1:
                vmeans = oracle.group_means(v[hi], labels[hi], C)
                np.testing.assert_array_equal(out["vbar"][hi].cpu().numpy(), vmeans.astype(np.float32))
                np.testing.assert_array_equal(out["Vp"][hi].float().cpu().numpy(), v[hi][perm])


@pytest.mark.parametrize("case", ["tiny", "ragged", "small"])
def test_kmeans_labels_and_centroids_match_oracle(case):
    torch = torch_gpu()
    w = CASES[case]
    log("kmeans %s" % case)
    data = upload(w)
    H = len(data["heads"])
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    q, k, v, iq, ik = data["host"]
    for side, X, Xh, C, init in ((0, data["Q"], q, w.Cq, iq), (1, data["K"], k, w.Ck, ik)):
        out = dict(labels=torch.empty(H, X.shape[1], dtype=torch.int32, device="cuda"),
                   cent=torch.empty(H, C, w.d, device="cuda"),
                   counts=torch.empty(H, C, dtype=torch.int32, device="cuda"),
                   offsets=torch.empty(H, C + 1, dtype=torch.int32, device="cuda"),
                   perm=torch.empty(H, X.shape[1], dtype=torch.int32, device="cuda"),
                   inv_perm=torch.empty(H, X.shape[1], dtype=torch.int32, device="cuda"),
                   Xp=torch.empty_like(X))
        V = None
        if side == 1:
            out["vbar"] = torch.empty(H, C, w.d, device="cuda")
            out["Vp"] = torch.empty_like(data["V"])
            V = data["V"]
        sv.cluster(shape, side, X, _dev(init, torch.int32), out, ws, V=V, flags=sv.DEBUG_SYNC)
        for hi in range(H):
            lab, cent, counts = oracle.kmeans(Xh[hi], C, init[hi], iters=w.iters)
            np.testing.assert_array_equal(out["labels"][hi].cpu().numpy(), lab)
            np.testing.assert_array_equal(out["counts"][hi].cpu().numpy(), counts)
            np.testing.assert_array_equal(out["cent"][hi].cpu().numpy(), cent.astype(np.float32))
            # the reorder: a stable sort by label, rows gathered in that order
            perm = oracle.permutation(lab, C)[2]
            np.testing.assert_array_equal(out["perm"][hi].cpu().numpy(), perm)
            np.testing.assert_array_equal(out["Xp"][hi].float().cpu().numpy(), Xh[hi][perm])
            if side == 1:
                np.testing.assert_array_equal(out["Vp"][hi].float().cpu().numpy(), v[hi][perm])


# ----------------------------------------------------------------------------- steps 2-3

def _probe_inputs(w, data, refs):
    """Oracle clustering as device tensors (centroids rounded to fp32 as the ABI takes them)."""
    torch = torch_gpu()
    q, k, v, iq, ik = data["host"]
    H = len(refs)
    f32 = lambda key: np.stack([r[key] for r in refs]).astype(np.float32)  # noqa: E731
    Kp = np.stack([k[h][refs[h]["perm_k"]] for h in range(H)])
    Vp = np.stack([v[h][refs[h]["perm_k"]] for h in range(H)])
    return dict(qbar=_dev(f32("qbar"), torch.float32), counts_q=_dev(np.stack([r["counts_q"] for r in refs]), torch.int32),
                Kp=_dev(Kp, _et(w)), Vp=_dev(Vp, _et(w)), kbar=_dev(f32("kbar"), torch.float32),
                vbar=_dev(f32("vbar"), torch.float32),
                counts_k=_dev(np.stack([r["counts_k"] for r in refs]), torch.int32),
                offsets_k=_dev(np.stack([r["offsets_k"] for r in refs]), torch.int32),
                Kp_h=Kp, Vp_h=Vp)


@pytest.mark.parametrize("case", ["tiny", "ragged", "small"])
def test_probe_ratios_and_eps_match_oracle(case):
    torch = torch_gpu()
    w = CASES[case]
    log("probe %s" % case)
    data = upload(w)
    refs = _oracle_all(w, data, w.rhos[0])
    H = len(refs)
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    P = _probe_inputs(w, data, refs)
    lr = torch.empty(H, w.Cq, w.Ck, device="cuda")
    le = torch.empty(H, w.Cq, w.N, device="cuda")
    sv.probe(shape, P["qbar"], P["counts_q"], P["Kp"], P["Vp"], P["kbar"], P["vbar"], P["counts_k"],
             P["offsets_k"], lr, ws, log_eps2=le, flags=sv.DEBUG_SYNC)
    for h in range(H):
        r = refs[h]
        qbar32, kbar32, vbar32 = (r[x].astype(np.float32).astype(np.float64) for x in ("qbar", "kbar", "vbar"))
        k64 = data["host"][1][h].astype(np.float64)
        v64 = data["host"][2][h].astype(np.float64)
        lratio, leps = oracle.probe_log(qbar32, r["counts_q"], k64, v64, r["labels_k"], kbar32, vbar32,
                                        r["counts_k"], want_eps=True)
        lfloor_blk, lfloor_key = probe_log_floors(qbar32, kbar32, vbar32, k64, v64, r["labels_k"], r["counts_k"])
        bad, dev = log_close(lr[h].cpu().numpy(), lratio, lfloor_blk)
        assert not bad.any(), (h, int(bad.sum()), float(dev[bad].max()))
        # per-key estimate, reordered key order
        badj, devj = log_close(le[h].cpu().numpy(), leps[:, r["perm_k"]], lfloor_key[:, r["perm_k"]])
        assert not badj.any(), (h, int(badj.sum()), float(devj[badj].max()))
        log("  head %d: max ratio dev %.2e, max eps dev %.2e" % (h, float(dev.max()), float(devj.max())))


@pytest.mark.parametrize("case", ["ragged", "small"])
def test_probe_repeats_bit_for_bit(case):
    """The probe hands key clusters to workgroups at run time (per-head claim
    counters); a cluster's estimate must not depend on which workgroup took it
    or when: repeated calls agree bit for bit."""
    torch = torch_gpu()
    w = CASES[case]
    log("probe repeatability %s" % case)
    data = upload(w)
    refs = _oracle_all(w, data, w.rhos[0])
    H = len(refs)
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    P = _probe_inputs(w, data, refs)
    outs = []
    for rep in range(8):
        lr = torch.empty(H, w.Cq, w.Ck, device="cuda")
        sv.probe(shape, P["qbar"], P["counts_q"], P["Kp"], P["Vp"], P["kbar"], P["vbar"], P["counts_k"],
                 P["offsets_k"], lr, ws)
        outs.append(lr.cpu())
    for rep in range(1, 8):
        assert torch.equal(outs[rep], outs[0]), "call %d differs from call 0" % rep


@pytest.mark.parametrize("case", ["tiny", "ragged", "small"])
def test_probe_logit_only_matches_oracle(case):
    """The logit-only estimate (SVGEAR_PROBE_LOGIT) against the oracle's, with the
    floor built from unit values (the estimate has no value terms)."""
    torch = torch_gpu()
    w = CASES[case]
    log("probe logit-only %s" % case)
    data = upload(w)
    refs = _oracle_all(w, data, w.rhos[0])
    H = len(refs)
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    P = _probe_inputs(w, data, refs)
    lr = torch.empty(H, w.Cq, w.Ck, device="cuda")
    le = torch.empty(H, w.Cq, w.N, device="cuda")
    sv.probe(shape, P["qbar"], P["counts_q"], P["Kp"], P["Vp"], P["kbar"], P["vbar"], P["counts_k"],
             P["offsets_k"], lr, ws, log_eps2=le, flags=sv.DEBUG_SYNC | sv.PROBE_LOGIT)
    for h in range(H):
        r = refs[h]
        qbar32, kbar32, vbar32 = (r[x].astype(np.float32).astype(np.float64) for x in ("qbar", "kbar", "vbar"))
        k64 = data["host"][1][h].astype(np.float64)
        v64 = data["host"][2][h].astype(np.float64)
        lratio, leps = oracle.probe_log(qbar32, r["counts_q"], k64, v64, r["labels_k"], kbar32, vbar32,
                                        r["counts_k"], want_eps=True, logit_only=True)
        unit_c = np.zeros_like(vbar32)
        unit_c[:, 0] = 1.0
        unit_k = np.zeros_like(v64)
        unit_k[:, 0] = 1.0
        lfb, lfk = probe_log_floors(qbar32, kbar32, unit_c, k64, unit_k, r["labels_k"], r["counts_k"])
        # Without value terms, e = a^2 expm1(D)^2 carries the absolute error of D
        # itself (the split-bf16 products are good to about 2^-16 of
        # tau sum_t |qbar_t delta_t|), squared-amplified where D is small: the bar
        # is 3e-3 for block means and 1e-2 per key (1e-3 for the value-aware probe).
        bad, dev = log_close(lr[h].cpu().numpy(), lratio, lfb, rtol=3e-3)
        assert not bad.any(), (h, int(bad.sum()), float(dev[bad].max()))
        badj, devj = log_close(le[h].cpu().numpy(), leps[:, r["perm_k"]], lfk[:, r["perm_k"]], rtol=1e-2)
        assert not badj.any(), (h, int(badj.sum()), float(devj[badj].max()))
        log("  head %d: max ratio dev %.2e, max eps dev %.2e" % (h, float(dev.max()), float(devj.max())))


def _route_gpu(w, H, lr, cq, ck, rho):
    torch = torch_gpu()
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    mask = torch.empty(H, w.Cq, w.Ck, dtype=torch.uint8, device="cuda")
    sel = torch.empty(H, dtype=torch.int64, device="cuda")
    sv.route(shape, rho, lr, cq, ck, mask, sel, ws)
    torch.cuda.synchronize()
    return mask.cpu().numpy(), sel.cpu().numpy()


@pytest.mark.parametrize("case", ["tiny", "ragged", "small"])
def test_route_mask_bit_exact_given_ratios(case):
    torch = torch_gpu()
    w = CASES[case]
    log("route %s" % case)
    rng = np.random.default_rng(7)
    H = 4
    cq = rng.integers(0, 2 * w.N // w.Cq, (H, w.Cq)).astype(np.int32)
    ck = rng.integers(0, 2 * w.N // w.Ck, (H, w.Ck)).astype(np.int32)
    cq[:, 0] = 0   # an empty query cluster
    ck[:, 1] = 0   # an empty key cluster
    variants = {
        "continuous": rng.standard_normal((H, w.Cq, w.Ck)).astype(np.float32) * 5,
        "ties": rng.integers(-3, 3, (H, w.Cq, w.Ck)).astype(np.float32),
        "with_-inf": np.where(rng.random((H, w.Cq, w.Ck)) < 0.2, -np.inf,
                              rng.standard_normal((H, w.Cq, w.Ck))).astype(np.float32),
    }
    Nq, Nk = int(cq[0].sum()), int(ck[0].sum())
    for name, lr in variants.items():
        for rho in (0.0, 0.05, w.rhos[0], 0.5, 1.0):
            # the budget uses the shape's Nq, Nk
            m, s = _route_gpu(w, H, _dev(lr, torch.float32), _dev(cq, torch.int32), _dev(ck, torch.int32), rho)
            for h in range(H):
                ref, used = oracle.route(lr[h].astype(np.float64), cq[h], ck[h], rho, w.N, w.N)
                np.testing.assert_array_equal(m[h], ref, err_msg="%s rho=%s head %d" % (name, rho, h))
                assert s[h] == used
    del Nq, Nk


@pytest.mark.parametrize("Cq,Ck,N", [(100, 500, 75600), (200, 1000, 118800), (64, 4096, 65536),
                                     (128, 4096, 65536)])
def test_route_mask_bit_exact_at_full_block_counts(Cq, Ck, N):
    """The head-wide route at the block counts of the Wan and HunyuanVideo
    shapes (50,000 and 200,000 blocks), at 2^18 blocks (five radix passes, a
    two-bit top digit), all three in two launches, and beyond 2^18 (524,288:
    one launch per pass): mask and selected cost bit-exact against the oracle.
    Tied ratios put more blocks on one 24-bit key prefix than the head
    workgroup keeps in LDS, so its later passes sweep the words and ratios
    again; continuous ratios keep those blocks in LDS."""
    torch = torch_gpu()
    log("route Cq=%d Ck=%d" % (Cq, Ck))
    rng = np.random.default_rng(Cq + Ck)
    H = 2
    cq = rng.integers(0, 2 * N // Cq + 1, (H, Cq)).astype(np.int32)
    ck = rng.integers(0, 2 * N // Ck + 1, (H, Ck)).astype(np.int32)
    cq[:, 0] = 0
    ck[:, 1] = 0
    variants = {
        "continuous": rng.standard_normal((H, Cq, Ck)).astype(np.float32) * 5,
        "ties": rng.integers(-3, 3, (H, Cq, Ck)).astype(np.float32),
        "with_-inf": np.where(rng.random((H, Cq, Ck)) < 0.2, -np.inf,
                              rng.standard_normal((H, Cq, Ck))).astype(np.float32),
    }
    shape = sv.make_shape(H, N, N, 128, Cq, Ck, 10, sv.BF16)
    ws = sv.alloc_workspace(shape)
    mask = torch.empty(H, Cq, Ck, dtype=torch.uint8, device="cuda")
    sel = torch.empty(H, dtype=torch.int64, device="cuda")
    for name, lr in variants.items():
        for rho in (0.0, 0.1, 0.15, 0.5, 1.0):
            sv.route(shape, rho, _dev(lr, torch.float32), _dev(cq, torch.int32), _dev(ck, torch.int32),
                     mask, sel, ws)
            torch.cuda.synchronize()
            m, st = mask.cpu().numpy(), sel.cpu().numpy()
            for h in range(H):
                ref, used = oracle.route(lr[h].astype(np.float64), cq[h], ck[h], rho, N, N)
                np.testing.assert_array_equal(m[h], ref, err_msg="%s rho=%s head %d" % (name, rho, h))
                assert st[h] == used, (name, rho, h)


@pytest.mark.parametrize("Cq,Ck", [(1, 1), (1, 7), (5, 1), (3, 5), (1, 4096), (4096, 1)])
def test_route_degenerate_block_grids(Cq, Ck):
    """Single blocks, single rows and columns and odd block counts (words past
    the last block in the last 16-byte vector, one key cluster per row so that
    the per-vector cluster stepping wraps several times): mask and selected
    cost bit-exact against the oracle, from rho = 0 to 1."""
    torch = torch_gpu()
    log("route grid %d x %d" % (Cq, Ck))
    rng = np.random.default_rng(Cq * 7 + Ck)
    H, N = 3, 4096
    cq = rng.integers(0, 2 * N // Cq + 2, (H, Cq)).astype(np.int32)
    ck = rng.integers(0, 2 * N // Ck + 2, (H, Ck)).astype(np.int32)
    variants = {
        "continuous": rng.standard_normal((H, Cq, Ck)).astype(np.float32) * 5,
        "ties": rng.integers(-1, 1, (H, Cq, Ck)).astype(np.float32),
    }
    shape = sv.make_shape(H, N, N, 128, Cq, Ck, 10, sv.BF16)
    ws = sv.alloc_workspace(shape)
    mask = torch.empty(H, Cq, Ck, dtype=torch.uint8, device="cuda")
    sel = torch.empty(H, dtype=torch.int64, device="cuda")
    for name, lr in variants.items():
        for rho in (0.0, 0.01, 0.3, 0.7, 1.0):
            sv.route(shape, rho, _dev(lr, torch.float32), _dev(cq, torch.int32), _dev(ck, torch.int32),
                     mask, sel, ws)
            torch.cuda.synchronize()
            m, st = mask.cpu().numpy(), sel.cpu().numpy()
            for h in range(H):
                ref, used = oracle.route(lr[h].astype(np.float64), cq[h], ck[h], rho, N, N)
                np.testing.assert_array_equal(m[h], ref, err_msg="%s rho=%s head %d" % (name, rho, h))
                assert st[h] == used, (name, rho, h)


@pytest.mark.parametrize("Cq,Ck,N", [(8, 16, 256), (13, 37, 1380), (64, 256, 8192), (3, 4096, 8192)])
def test_route_rows_bit_exact_given_ratios(Cq, Ck, N):
    """Per-query-cluster budgets: mask and total cost bit-exact against the
    oracle on continuous, tied and partly -inf ratios, from rho = 0 to 1,
    including the largest key-cluster count (4096)."""
    torch = torch_gpu()
    log("route_rows Cq=%d Ck=%d" % (Cq, Ck))
    rng = np.random.default_rng(Cq * 1000 + Ck)
    H = 2
    cq = rng.integers(0, 2 * N // Cq + 1, (H, Cq)).astype(np.int32)
    ck = rng.integers(0, 2 * N // Ck + 1, (H, Ck)).astype(np.int32)
    cq[:, 0] = 0
    ck[:, 1] = 0
    variants = {
        "continuous": rng.standard_normal((H, Cq, Ck)).astype(np.float32) * 5,
        "ties": rng.integers(-3, 3, (H, Cq, Ck)).astype(np.float32),
        "with_-inf": np.where(rng.random((H, Cq, Ck)) < 0.2, -np.inf,
                              rng.standard_normal((H, Cq, Ck))).astype(np.float32),
    }
    shape = sv.make_shape(H, N, N, 128, Cq, Ck, 10, sv.BF16)
    ws = sv.alloc_workspace(shape)
    mask = torch.empty(H, Cq, Ck, dtype=torch.uint8, device="cuda")
    sel = torch.empty(H, dtype=torch.int64, device="cuda")
    for name, lr in variants.items():
        for rho in (0.0, 0.05, 0.3, 0.5, 1.0):
            sv.route_rows(shape, rho, _dev(lr, torch.float32), _dev(cq, torch.int32), _dev(ck, torch.int32),
                          mask, sel, ws)
            torch.cuda.synchronize()
            m, st = mask.cpu().numpy(), sel.cpu().numpy()
            for h in range(H):
                ref, used = oracle.route_rows(lr[h].astype(np.float64), cq[h], ck[h], rho, N)
                np.testing.assert_array_equal(m[h], ref, err_msg="%s rho=%s head %d" % (name, rho, h))
                assert st[h] == used


# ----------------------------------------------------------------------------- step 4

@pytest.mark.parametrize("case", ["tiny", "ragged", "small"])
@pytest.mark.parametrize("rho", [None, 0.0, 1.0])
def test_attention_matches_oracle_given_routing(case, rho):
    torch = torch_gpu()
    w = CASES[case]
    rho = w.rhos[0] if rho is None else rho
    log("attention %s rho=%s" % (case, rho))
    data = upload(w)
    refs = _oracle_all(w, data, rho)
    H = len(refs)
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    q, k, v = data["host"][:3]
    P = _probe_inputs(w, data, refs)
    Qp = np.stack([q[h][refs[h]["perm_q"]] for h in range(H)])
    O = torch.empty_like(data["Q"])
    sv.attention(shape, _dev(Qp, _et(w)), _dev(np.stack([r["offsets_q"] for r in refs]), torch.int32),
                 _dev(np.stack([r["perm_q"] for r in refs]), torch.int32), P["Kp"], P["Vp"], P["kbar"],
                 P["vbar"], P["counts_k"], P["offsets_k"], _dev(np.stack([r["mask"] for r in refs]), torch.uint8),
                 O, ws)
    torch.cuda.synchronize()
    O = O.float().cpu().numpy()
    for h in range(H):
        r = refs[h]
        ref = oracle.hybrid(q[h], k[h], v[h], r["labels_q"], r["labels_k"], r["kbar"].astype(np.float32),
                            r["vbar"].astype(np.float32), r["counts_k"], r["mask"])
        check_output(O[h], ref, w.dtype, "head %d" % h)


# ----------------------------------------------------------------------------- end to end

@pytest.mark.parametrize("case,rho", [("tiny", 0.25), ("tiny", 1.0), ("ragged", 0.3), ("small", 0.2)])
def test_forward_end_to_end(case, rho):
    w = CASES[case]
    log("forward %s rho=%s" % (case, rho))
    out, data = gpu_forward(w, rho)
    H = len(data["heads"])
    for h in range(H):
        r = oracle_head(w, data, h, rho)
        for key in ("labels_q", "counts_q", "offsets_q", "perm_q", "inv_perm_q", "labels_k", "counts_k",
                    "offsets_k", "perm_k", "inv_perm_k"):
            np.testing.assert_array_equal(out[key][h].numpy(), r[key], err_msg="%s head %d" % (key, h))
        nd = near_threshold_ok(out["mask"][h].numpy(), r["mask"], r["log_ratio"])
        if nd == 0:
            assert int(out["sel_cost"][h]) == int(r["sel_cost"])
        assert int(out["sel_cost"][h]) <= int(r["budget"])
        ref = r["O"]
        if nd:   # rows of query clusters whose mask row flipped: oracle with the library's mask
            q, k, v = (a[h] for a in data["host"][:3])
            ref, _ = reference_rows(q, k, v, r["labels_q"], r["labels_k"], r["kbar"], r["vbar"], r["counts_k"],
                                    r["mask"], out["mask"][h].numpy(), np.arange(w.N))
        check_output(out["O"][h], ref, w.dtype, "head %d O" % h)


def _cluster_given(w, shape, X, labels, C, ws, V=None):
    torch = torch_gpu()
    H, N = labels.shape
    out = dict(labels=_dev(labels, torch.int32), cent=torch.empty(H, C, w.d, device="cuda"),
               counts=torch.empty(H, C, dtype=torch.int32, device="cuda"),
               offsets=torch.empty(H, C + 1, dtype=torch.int32, device="cuda"),
               perm=torch.empty(H, N, dtype=torch.int32, device="cuda"),
               inv_perm=torch.empty(H, N, dtype=torch.int32, device="cuda"), Xp=torch.empty_like(X))
    if V is not None:
        out["vbar"] = torch.empty(H, C, w.d, device="cuda")
        out["Vp"] = torch.empty_like(V)
    sv.cluster(shape, 1 if V is not None else 0, X, None, out, ws, V=V, flags=sv.LABELS_GIVEN | sv.DEBUG_SYNC)
    return out


@pytest.mark.parametrize("case", ["tiny", "ragged"])
def test_probe_exact_special_cases(case):
    """Keys equal to their centroid: the estimate is exactly zero when the values
    are equal too (singleton clusters), and a^2 ||vbar - v||^2 otherwise."""
    torch = torch_gpu()
    w = CASES[case]
    log("probe special cases %s" % case)
    rng = np.random.default_rng(3)
    H, N, G = 2, 640, 40
    shape = sv.make_shape(H, N, N, w.d, 8, G, 2, sv.BF16 if w.dtype == "bf16" else sv.F32)
    ws = sv.alloc_workspace(shape)
    from sparse_attention_video_flash_amd.inputs import round_to_bf16
    rnd = round_to_bf16 if w.dtype == "bf16" else (lambda a: a.astype(np.float32))
    lab_k = rng.integers(0, G, (H, N)).astype(np.int32)
    lab_k[:, :G] = np.arange(G)                           # every cluster non-empty
    kc = rnd(rng.standard_normal((H, G, w.d)).astype(np.float32))
    K = np.stack([kc[h][lab_k[h]] for h in range(H)])    # keys identical within clusters
    V = rnd(rng.standard_normal((H, N, w.d)).astype(np.float32))
    qbar = rng.standard_normal((H, 8, w.d)).astype(np.float32)
    cq = np.full((H, 8), N // 8, np.int32)
    o = _cluster_given(w, shape, _dev(K, _et(w)), lab_k, G, ws, V=_dev(V, _et(w)))
    lr = torch.empty(H, 8, G, device="cuda")
    sv.probe(shape, _dev(qbar, torch.float32), _dev(cq, torch.int32), o["Xp"], o["Vp"], o["cent"], o["vbar"],
             o["counts"], o["offsets"], lr, ws, flags=sv.DEBUG_SYNC)
    lr = lr.cpu().numpy()
    for h in range(H):
        kbar = o["cent"][h].cpu().numpy().astype(np.float64)
        vbar = o["vbar"][h].cpu().numpy().astype(np.float64)
        ratio = oracle.probe(qbar[h], cq[h], K[h], V[h], lab_k[h], kbar, vbar, o["counts"][h].cpu().numpy())
        np.testing.assert_allclose(lr[h], np.log(ratio), rtol=0, atol=1e-4)
    # now values identical within clusters too: every estimate is exactly zero
    V2 = np.stack([V[h][:G][lab_k[h]] for h in range(H)])
    o = _cluster_given(w, shape, _dev(K, _et(w)), lab_k, G, ws, V=_dev(V2, _et(w)))
    lr2 = torch.empty(H, 8, G, device="cuda")
    sv.probe(shape, _dev(qbar, torch.float32), _dev(cq, torch.int32), o["Xp"], o["Vp"], o["cent"], o["vbar"],
             o["counts"], o["offsets"], lr2, ws, flags=sv.DEBUG_SYNC)
    assert (lr2.cpu().numpy() == -np.inf).all()


@pytest.mark.parametrize("case", ["ragged", "small"])
def test_forward_equals_stage_by_stage_path(case):
    """svgear_forward clusters Q on a side stream while K is clustered; its
    intermediates and output must equal those of the per-stage entry points run
    one after another on one stream, bit for bit, call after call."""
    torch = torch_gpu()
    w = CASES[case]
    log("forward vs stages %s" % case)
    data = upload(w)
    H = len(data["heads"])
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    rho = w.rhos[0]
    ref_im = sv.alloc_intermediates(shape)
    O_ref = torch.empty_like(data["Q"])
    im = ref_im
    sv.cluster(shape, 0, data["Q"], data["init_q"], dict(labels=im["labels_q"], cent=im["qbar"], counts=im["counts_q"],
                                                         offsets=im["offsets_q"], perm=im["perm_q"],
                                                         inv_perm=im["inv_perm_q"], Xp=im["Qp"]), ws)
    sv.cluster(shape, 1, data["K"], data["init_k"], dict(labels=im["labels_k"], cent=im["kbar"], vbar=im["vbar"],
                                                         counts=im["counts_k"], offsets=im["offsets_k"],
                                                         perm=im["perm_k"], inv_perm=im["inv_perm_k"], Xp=im["Kp"],
                                                         Vp=im["Vp"]), ws, V=data["V"])
    sv.probe(shape, im["qbar"], im["counts_q"], im["Kp"], im["Vp"], im["kbar"], im["vbar"], im["counts_k"],
             im["offsets_k"], im["log_ratio"], ws)
    sv.route(shape, rho, im["log_ratio"], im["counts_q"], im["counts_k"], im["mask"], im["sel_cost"], ws)
    sv.attention(shape, im["Qp"], im["offsets_q"], im["perm_q"], im["Kp"], im["Vp"], im["kbar"], im["vbar"],
                 im["counts_k"], im["offsets_k"], im["mask"], O_ref, ws)
    torch.cuda.synchronize()
    ref = {k: v.cpu() for k, v in ref_im.items()}
    for rep in range(3):
        im2 = sv.alloc_intermediates(shape)
        O = torch.empty_like(data["Q"])
        sv.forward(shape, rho, data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O, ws, im2)
        torch.cuda.synchronize()
        for k, v in im2.items():
            assert torch.equal(v.cpu(), ref[k]), "%s differs on call %d" % (k, rep)
        assert torch.equal(O.cpu(), O_ref.cpu()), "output differs on call %d" % rep


def test_forward_replays_from_a_hip_graph():
    """svgear_forward captured into a HIP graph (torch.cuda.graph) and replayed
    several times, with eager work and synchronisations in between: every
    replay equals the eager call bit for bit (the side-stream fork/join, the
    queue counters and every cleared buffer are graph-safe: kernels only)."""
    torch = torch_gpu()
    w = CASES["small"]
    log("forward under graph capture")
    data = upload(w)
    H = len(data["heads"])
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    rho = w.rhos[0]
    O_ref = torch.empty_like(data["Q"])
    sv.forward(shape, rho, data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O_ref, ws)
    torch.cuda.synchronize()
    ref = O_ref.cpu()
    O = torch.empty_like(data["Q"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.forward(shape, rho, data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O, ws)
    for rep in range(4):
        O.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O.cpu(), ref), "replay %d differs from the eager call" % rep
        # eager work between replays, on the same workspace
        sv.forward(shape, rho, data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O_ref, ws)
        torch.cuda.synchronize()
        assert torch.equal(O_ref.cpu(), ref)


@pytest.mark.parametrize("case", ["tiny", "ragged", "small"])
def test_forward_is_deterministic_over_stale_workspace(case):
    """The same inputs give bit-identical outputs and intermediates, whatever
    the workspace and the intermediate buffers held before the call: two calls
    over buffers filled with different random bytes agree exactly (nothing
    reads memory the call did not write first)."""
    torch = torch_gpu()
    w = CASES[case]
    log("forward determinism %s" % case)
    data = upload(w)
    H = len(data["heads"])
    shape = shape_of(w, H)
    rho = w.rhos[0]
    gen = torch.Generator(device="cuda")
    runs = []
    for seed in (1, 2):
        gen.manual_seed(seed)
        ws = sv.alloc_workspace(shape)
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=gen))
        im = sv.alloc_intermediates(shape, "cuda")
        for t in im.values():
            raw = t.view(torch.uint8)
            raw.copy_(torch.randint(0, 256, raw.shape, dtype=torch.uint8, device="cuda", generator=gen))
        O = torch.empty_like(data["Q"])
        O.view(torch.uint8).copy_(torch.randint(0, 256, O.view(torch.uint8).shape, dtype=torch.uint8,
                                                device="cuda", generator=gen))
        sv.forward(shape, rho, data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O, ws, im)
        torch.cuda.synchronize()
        runs.append(({k: v.cpu() for k, v in im.items()}, O.cpu()))
    (im1, O1), (im2, O2) = runs
    for k in im1:
        a, b = im1[k].view(torch.uint8), im2[k].view(torch.uint8)
        assert torch.equal(a, b), "intermediate %s differs between the two calls" % k
    assert torch.equal(O1.view(torch.uint8), O2.view(torch.uint8)), "output differs between the two calls"


def test_forward_on_two_streams_at_once():
    """Two svgear_forward calls with their own workspaces, enqueued back to back
    on two streams without a synchronisation in between (both share the
    library's side stream for the Q clustering): each equals the same call
    made alone."""
    torch = torch_gpu()
    wa, wb = CASES["small"], CASES["ragged"]
    log("forward on two streams")
    runs = []
    for w in (wa, wb):
        data = upload(w)
        H = len(data["heads"])
        shape = shape_of(w, H)
        runs.append((w, data, shape, sv.alloc_workspace(shape)))
    alone = []
    for w, data, shape, ws in runs:
        O = torch.empty_like(data["Q"])
        sv.forward(shape, w.rhos[0], data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O, ws)
        torch.cuda.synchronize()
        alone.append(O.cpu())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (w, data, shape, ws), st in zip(runs, streams):
        O = torch.empty_like(data["Q"])
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            sv.forward(shape, w.rhos[0], data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O, ws,
                       stream=st)
        outs.append(O)
    torch.cuda.synchronize()
    for ref, O in zip(alone, outs):
        assert torch.equal(O.cpu(), ref), "a call made beside another differs from the call made alone"
