"""svgear_probe_noalloc (the probe with its scratch in the library's own
per-device array, for callers that cannot allocate) against svgear_probe with
a caller workspace: the same kernels on the same inputs, so the ratios (and the
per-key debug output) must be bit-identical.  Two calls in a row, the second
on a smaller problem, so the second runs over the first one's leftovers; both
the MFMA path (bf16, d = 128) and the generic path (fp32, d = 64, which also
keeps per-key value terms in the array) are covered."""
import numpy as np
import pytest

from sparse_attention_video_flash_amd import svgear as sv
from sparse_attention_video_flash_amd.inputs import WORKLOADS, Mixture, Workload

from gpu_common import RAGGED, log, shape_of, torch_gpu, upload

pytestmark = pytest.mark.gpu

FLAGS = {"error": 0, "logit": sv.PROBE_LOGIT, "score": sv.PROBE_SCORE, "eps": sv.DEBUG_EPS}


def _clustered(w):
    """One forward (all intermediates kept) to get a real clustering."""
    torch = torch_gpu()
    data = upload(w)
    H = len(data["heads"])
    shape = shape_of(w, H)
    ws = sv.alloc_workspace(shape)
    im = sv.alloc_intermediates(shape)
    O = torch.empty_like(data["Q"])
    sv.forward(shape, w.rhos[0], data["Q"], data["K"], data["V"], data["init_q"], data["init_k"], O, ws, im)
    return shape, ws, im


def _both(shape, ws, im, flags):
    torch = torch_gpu()
    H, Cq, Ck, Nk = shape.H, shape.Cq, shape.Ck, shape.Nk
    out = []
    for noalloc in (False, True):
        lr = torch.full((H, Cq, Ck), float("nan"), device="cuda")
        le = torch.full((H, Cq, Nk), float("nan"), device="cuda") if flags & sv.DEBUG_EPS else None
        args = (shape, im["qbar"], im["counts_q"], im["Kp"], im["Vp"], im["kbar"], im["vbar"], im["counts_k"],
                im["offsets_k"], lr)
        if noalloc:
            sv.probe_noalloc(*args, log_eps2=le, flags=flags & ~sv.DEBUG_EPS)
        else:
            sv.probe(*args[:-1], lr, ws, log_eps2=le, flags=flags & ~sv.DEBUG_EPS)
        torch.cuda.synchronize()
        out.append((lr.cpu().numpy(), None if le is None else le.cpu().numpy()))
    return out


# fp32, d = 64, two heads of 1380 tokens: larger than the tiny workload
GENERIC = Workload("generic", 2, (3, 20, 23), 64, "fp32", 9, 41, 10, (0.3,), 13,
                   (Mixture((0, 2), 24, (2, 3, 4), 0.25, "normal", 0.08, 2.0, "add"),))
CASES = {"small": WORKLOADS["small"], "ragged": RAGGED, "generic": GENERIC, "tiny": WORKLOADS["tiny"]}


@pytest.mark.parametrize("first,second", [("small", "ragged"), ("generic", "tiny")])
def test_probe_noalloc_matches_probe(first, second):
    for name in (first, second):   # the second call is the smaller problem
        w = CASES[name]
        shape, ws, im = _clustered(w)
        for mode, flags in FLAGS.items():
            (lr_ws, le_ws), (lr_na, le_na) = _both(shape, ws, im, flags)
            np.testing.assert_array_equal(lr_na, lr_ws, err_msg="%s %s" % (name, mode))
            assert not np.isnan(lr_na).any()
            if le_ws is not None:
                np.testing.assert_array_equal(le_na, le_ws, err_msg="%s %s eps" % (name, mode))
            log("noalloc %s (%d heads, Cq=%d, Ck=%d) %s: bit-identical" % (name, shape.H, shape.Cq, shape.Ck, mode))
