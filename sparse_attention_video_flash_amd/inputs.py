"""Seeded synthetic inputs for one routed attention call.

This module holds the workload definitions and the random-number recipe that both
the HIP path and the fp64 oracle consume.  It contains none of the method's
arithmetic: it only draws Gaussian-mixture Q/K/V tensors shaped like the video
workloads of the SVG-EAR pages (Wan2.2 and HunyuanVideo latent grids, 720p), and
the k-means initial indices, which the method draws at random and which are
therefore passed in as data.

Recipe (per head h, each head from its own stream so heads can be drawn
independently and in parallel):

* ``rng = numpy.random.default_rng([seed, h])``
* component means ``(M, d) ~ N(0, I)`` (float64, then used in float32)
* for X in (Q, K, V), in that order:
  noise ``(N, d)`` standard normal (float32; Student-t(3) for heavy-tailed heads),
  then, if the workload has outliers, a Bernoulli mask ``(N,)`` (uniform < frac)
  and outlier noise ``(count, d)`` for the masked tokens only.
* token ``n = (t*Hg + y)*Wg + x`` on the ``T x Hg x Wg`` latent grid; its
  component is ``(floor(t*Pt/T)*Py + floor(y*Py/Hg))*Px + floor(x*Px/Wg)``:
  contiguous spatio-temporal boxes, each with its own mean.
* Q, K and V share a head's component means; their noise is independent.
* bf16 workloads round the float32 values to bf16 (round to nearest even), so
  the float32 arrays returned here are exactly representable in bf16.
* init indices: ``default_rng([seed, 1000 + h])``: ``choice(Nq, Cq)`` then
  ``choice(Nk, Ck)``, without replacement, as int32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Mixture:
    """Gaussian-mixture recipe for a range of heads."""

    heads: Tuple[int, int]            # [first, last) head index
    components: int                   # number of mixture components M
    patches: Tuple[int, int, int]     # (Pt, Py, Px); Pt*Py*Px == components
    sigma: float                      # token noise scale
    noise: str = "normal"             # "normal" or "student_t3"
    outlier_frac: float = 0.0
    outlier_sigma: float = 0.0
    outlier_mode: str = "none"        # "replace": N(0, s^2 I); "add": mean + N(0, s^2 I)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    grid: Tuple[int, int, int]        # (T, Hg, Wg) latent grid
    d: int
    dtype: str                        # "fp32" or "bf16"
    Cq: int
    Ck: int
    iters: int
    rhos: Tuple[float, ...]
    seed: int
    mixtures: Tuple[Mixture, ...]

    @property
    def N(self) -> int:
        t, y, x = self.grid
        return t * y * x

    def mixture_for(self, h: int) -> Mixture:
        for m in self.mixtures:
            if m.heads[0] <= h < m.heads[1]:
                return m
        raise KeyError(h)


WORKLOADS: Dict[str, Workload] = {
    # 1 head, 1024 tokens, d=64, fp32; 16 components in 4x4x4 boxes.
    "tiny": Workload("tiny", 1, (4, 16, 16), 64, "fp32", 8, 16, 10, (0.25, 1.0), 0,
                     (Mixture((0, 1), 16, (1, 4, 4), 0.3),)),
    # 8 heads, 8192 tokens; 10% outliers replaced by N(0, 4I).
    "small": Workload("small", 8, (8, 32, 32), 128, "bf16", 64, 256, 10, (0.2,), 1,
                      (Mixture((0, 8), 64, (4, 4, 4), 0.25, "normal", 0.10, 2.0, "replace"),)),
    # Wan2.2-shaped: 40 heads x 75,600 tokens (21x45x80).
    "wan": Workload("wan", 40, (21, 45, 80), 128, "bf16", 100, 500, 10, (0.15,), 2,
                    (Mixture((0, 40), 400, (4, 10, 10), 0.2, "normal", 0.05, 2.0, "add"),)),
    # HunyuanVideo-shaped: 24 heads x 118,800 tokens (33x45x80).
    "hunyuan": Workload("hunyuan", 24, (33, 45, 80), 128, "bf16", 200, 1000, 10, (0.10,), 3,
                        (Mixture((0, 24), 800, (8, 10, 10), 0.2, "normal", 0.05, 2.0, "add"),)),
    # Routing stress: tight mixture on heads 0-7, heavy-tailed standard Student-t(3) noise
    # (unit scale; values reach a few hundred) on heads 8-15.
    "stress": Workload("stress", 16, (8, 64, 64), 128, "bf16", 128, 512, 10,
                       (0.05, 0.1, 0.25, 0.5, 1.0), 4,
                       (Mixture((0, 8), 256, (4, 8, 8), 0.1),
                        Mixture((8, 16), 64, (4, 4, 4), 1.0, "student_t3"))),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def component_of_tokens(grid: Tuple[int, int, int], patches: Tuple[int, int, int]) -> np.ndarray:
    """Mixture component of every token of the latent grid, in token order."""
    T, Hg, Wg = grid
    Pt, Py, Px = patches
    t = np.arange(T)[:, None, None]
    y = np.arange(Hg)[None, :, None]
    x = np.arange(Wg)[None, None, :]
    comp = ((t * Pt // T) * Py + (y * Py // Hg)) * Px + (x * Px // Wg)
    return comp.reshape(-1).astype(np.int64)


def _draw_tensor(rng: np.random.Generator, means: np.ndarray, comp: np.ndarray,
                 mix: Mixture, N: int, d: int) -> np.ndarray:
    if mix.noise == "normal":
        noise = rng.standard_normal((N, d), dtype=np.float32)
    elif mix.noise == "student_t3":
        noise = rng.standard_t(3.0, size=(N, d)).astype(np.float32)
    else:
        raise ValueError(mix.noise)
    x = means[comp] + np.float32(mix.sigma) * noise
    if mix.outlier_frac > 0.0:
        sel = rng.random(N) < mix.outlier_frac
        cnt = int(sel.sum())
        extra = np.float32(mix.outlier_sigma) * rng.standard_normal((cnt, d), dtype=np.float32)
        if mix.outlier_mode == "replace":
            x[sel] = extra
        elif mix.outlier_mode == "add":
            x[sel] = means[comp[sel]] + extra
        else:
            raise ValueError(mix.outlier_mode)
    return x


def generate_head(w: Workload, h: int, Nq: Optional[int] = None, Nk: Optional[int] = None):
    """Draw (Q, K, V, init_q, init_k) for head ``h`` of workload ``w``.

    Q: (Nq, d), K and V: (Nk, d) float32 (bf16-representable for bf16 workloads);
    init_q: (Cq,), init_k: (Ck,) int32.
    """
    N = w.N
    Nq = N if Nq is None else Nq
    Nk = N if Nk is None else Nk
    mix = w.mixture_for(h)
    rng = np.random.default_rng([w.seed, h])
    means = rng.standard_normal((mix.components, w.d)).astype(np.float32)
    comp = component_of_tokens(w.grid, mix.patches)
    out = []
    for n in (Nq, Nk, Nk):
        x = _draw_tensor(rng, means, comp[:n] if n <= N else np.resize(comp, n), mix, n, w.d)
        if w.dtype == "bf16":
            x = round_to_bf16(x)
        out.append(np.ascontiguousarray(x, dtype=np.float32))
    irng = np.random.default_rng([w.seed, 1000 + h])
    init_q = irng.choice(Nq, size=w.Cq, replace=False).astype(np.int32)
    init_k = irng.choice(Nk, size=w.Ck, replace=False).astype(np.int32)
    return out[0], out[1], out[2], init_q, init_k


def generate(w: Workload, heads: Optional[Sequence[int]] = None):
    """Stack ``generate_head`` over ``heads`` (default: all): arrays [h, N, d] and [h, C]."""
    heads = list(range(w.H)) if heads is None else list(heads)
    parts = [generate_head(w, h) for h in heads]
    return tuple(np.stack([p[i] for p in parts]) for i in range(5))


__all__: List[str] = ["Mixture", "Workload", "WORKLOADS", "round_to_bf16", "component_of_tokens",
                      "generate_head", "generate"]
