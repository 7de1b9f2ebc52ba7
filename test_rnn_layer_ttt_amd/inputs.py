"""Seeded synthetic inputs for the TTT-Linear scan.

This module only draws and rounds random numbers; it holds none of the
scan's arithmetic, so that the GPU path and the CPU oracle can both be fed
from it without sharing any code of the method.

The workloads have the shapes the pages use: d = 64 inner heads
("Edifice.Recurrent.TTT": ``inner_size`` 64, hidden a multiple of it, heads =
hidden / inner) over long sequences, with W0 ~ N(0, 0.02) (standard
deviation 0.02, "Paper-Faithful Implementation" item 1).  No dataset or
trained weight is involved: every value is synthetic.

Recipe: ``numpy.random.Generator(PCG64(seed))``; draw order W0, q, k, v,
eta_logit, gate_logit, then gamma and beta when they are random; each draw
is ``standard_normal(dtype=float32)`` of the full array shape; affine maps
and the optional per-token L2 normalisation are done in float64 and cast
back to float32 (round to nearest even).  For bf16 workloads q, k, v,
eta_logit and gate_logit are then rounded float32 -> bf16 (round to nearest
even) and handed out as float32 arrays that hold exactly the bf16 values,
so that the oracle and the GPU see identical numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class ScanInputs:
    """One seeded problem.  All arrays are float32 and C-contiguous."""
    name: str
    q: np.ndarray          # [B,H,T,d]
    k: np.ndarray          # [B,H,T,d]
    v: np.ndarray          # [B,H,T,d]
    eta_logit: np.ndarray  # [B,H,T]
    gate_logit: np.ndarray  # [B,H,T,d]
    W0: np.ndarray         # [B,H,d,d]
    gamma: np.ndarray      # [H,d]
    beta: np.ndarray       # [H,d]
    ln: str = "st"         # "st" | "exact" | "none"
    dual: bool = False
    chunk: int = 16
    in_bf16: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        return self.q.shape

    def subset(self, pairs):
        """The same problem restricted to a list of (b, h) scans, stacked as B=1, H=len."""
        bs = [p[0] for p in pairs]
        hs = [p[1] for p in pairs]
        sel = lambda a: np.ascontiguousarray(a[bs, hs][None])
        return ScanInputs(
            name=self.name + "[subset]", q=sel(self.q), k=sel(self.k), v=sel(self.v),
            eta_logit=sel(self.eta_logit), gate_logit=sel(self.gate_logit), W0=sel(self.W0),
            gamma=np.ascontiguousarray(self.gamma[hs]),
            beta=np.ascontiguousarray(self.beta[hs]),
            ln=self.ln, dual=self.dual, chunk=self.chunk, in_bf16=self.in_bf16,
            meta=dict(self.meta, subset=list(pairs)))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _f32(a64: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a64.astype(np.float32))


def make_case(B: int, H: int, T: int, d: int, seed: int, *, ln: str = "st",
              dual: bool = False, chunk: int = 16, in_bf16: bool = False,
              l2norm_qkv: bool = False, random_affine: bool = False,
              eta_mean: float = 0.0, w0_std: float = 0.02, v_mean: float = 0.0,
              w0_common_row: float = 0.0, name: str | None = None) -> ScanInputs:
    """Draw one problem following the recipe in the module docstring.

    Off-centre LayerNorm inputs (both off by default, and drawn after
    everything else so that the other draws do not change): ``v_mean`` adds a
    constant to every v (the targets, so the inner model's outputs drift to a
    large common mean), and ``w0_common_row`` adds ``w0_common_row * r`` to
    every row of W0, r ~ N(0,1)^d / sqrt(d) (so z = W0 k starts with a common
    component r.k, large against its spread across the features)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    draw = lambda *shape: rng.standard_normal(shape, dtype=np.float32)
    W0 = _f32(draw(B, H, d, d).astype(np.float64) * w0_std)
    q, k, v = draw(B, H, T, d), draw(B, H, T, d), draw(B, H, T, d)
    eta = draw(B, H, T)
    if eta_mean != 0.0:
        eta = _f32(eta.astype(np.float64) + eta_mean)
    gate = draw(B, H, T, d)
    if random_affine:
        gamma = _f32(1.0 + 0.1 * draw(H, d).astype(np.float64))
        beta = _f32(0.1 * draw(H, d).astype(np.float64))
    else:
        gamma = np.ones((H, d), np.float32)
        beta = np.zeros((H, d), np.float32)
    if l2norm_qkv:
        def nrm(a):
            a64 = a.astype(np.float64)
            return _f32(a64 / np.linalg.norm(a64, axis=-1, keepdims=True) * np.sqrt(d))
        q, k, v = nrm(q), nrm(k), nrm(v)
    if v_mean != 0.0:
        v = _f32(v.astype(np.float64) + v_mean)
    if w0_common_row != 0.0:
        r = draw(B, H, 1, d).astype(np.float64) / np.sqrt(d)
        W0 = _f32(W0.astype(np.float64) + w0_common_row * r)
    if in_bf16:
        q, k, v, eta, gate = (round_to_bf16(a) for a in (q, k, v, eta, gate))
    return ScanInputs(name=name or f"B{B}_H{H}_T{T}_d{d}", q=q, k=k, v=v, eta_logit=eta,
                      gate_logit=gate, W0=W0, gamma=gamma, beta=beta, ln=ln, dual=dual,
                      chunk=chunk, in_bf16=in_bf16,
                      meta=dict(B=B, H=H, T=T, d=d, seed=seed, l2norm_qkv=l2norm_qkv,
                                random_affine=random_affine, eta_mean=eta_mean, v_mean=v_mean,
                                w0_common_row=w0_common_row))


#: The five named workloads.  Sizes, distributions and seeds are the ones the
#: scan is specified on; hidden = H * d.
WORKLOADS = {
    # per-token, fp32, tiny: the case the oracle finishes in well under a second
    "tiny_d16_fp32": dict(B=1, H=2, T=64, d=16, seed=0),
    # per-token, fp32, hidden 256, unit-norm*sqrt(d) q/k/v, random LN affine
    "h256_T2048_fp32": dict(B=8, H=4, T=2048, d=64, seed=1, l2norm_qkv=True,
                            random_affine=True),
    # per-token, bf16 inputs, hidden 1024, 256 scans
    "h1024_T4096_bf16": dict(B=16, H=16, T=4096, d=64, seed=2, in_bf16=True),
    # dual form, chunk 16, bf16 inputs, hidden 2048, 256 scans
    "h2048_T8192_dual16_bf16": dict(B=8, H=32, T=8192, d=64, seed=3, in_bf16=True,
                                    dual=True, chunk=16),
    # exact LayerNorm-Jacobian inner gradient, fp32, hidden 2048, 128 scans
    "h2048_T16384_exact_fp32": dict(B=4, H=32, T=16384, d=64, seed=4, ln="exact",
                                    random_affine=True, eta_mean=-1.0),
}


def make_inputs(workload: str, **overrides) -> ScanInputs:
    """Draw one of the named workloads (keyword overrides change its fields)."""
    cfg = dict(WORKLOADS[workload])
    cfg.update(overrides)
    return make_case(name=workload, **cfg)


def make_cotangents(B: int, H: int, T: int, d: int, seed: int, *, with_state: bool = True):
    """Seeded loss gradients for a backward pass: ``(dout, dW_final)``, float32,
    dout [B,H,T,d] ~ N(0,1) and dW_final [B,H,d,d] ~ N(0,1) (or None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dout = rng.standard_normal((B, H, T, d), dtype=np.float32)
    dWf = rng.standard_normal((B, H, d, d), dtype=np.float32) if with_state else None
    return dout, dWf


def make_update_mask(B: int, H: int, T: int, chunk: int, rate: float, seed: int) -> np.ndarray:
    """Seeded SKIP (0) / UPDATE (1) decisions, one per chunk: uint8
    [B,H,ceil(T/chunk)], each 1 with probability ``rate``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = -(-T // chunk) if T > 0 else 0
    return (rng.random((B, H, n)) < rate).astype(np.uint8)


def make_projection_case(B: int, T: int, hidden: int, H: int, d: int, seed: int, *,
                         with_bias: bool = False):
    """Seeded input of the layer's input projections: ``(x, w_proj, b_proj)``.

    x [B,T,hidden] ~ N(0,1) and w_proj [H,4d+1,hidden] ~ N(0, 1/hidden) (so
    that each projection is ~ N(0,1), the scale of the scan's own inputs),
    both rounded to bf16 (nearest even) and handed out as float32 holding the
    bf16 values; b_proj [H,4d+1] ~ N(0, 0.1^2) in float32, or None.  Draw
    order x, w_proj, b_proj.  The rows of one head are stacked q (d), k (d),
    v (d), gate (d), eta (1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = round_to_bf16(rng.standard_normal((B, T, hidden), dtype=np.float32))
    w = rng.standard_normal((H, 4 * d + 1, hidden), dtype=np.float32)
    w = round_to_bf16(_f32(w.astype(np.float64) / np.sqrt(hidden)))
    b = None
    if with_bias:
        b = _f32(rng.standard_normal((H, 4 * d + 1), dtype=np.float32).astype(np.float64) * 0.1)
    return x, w, b


def make_mlp_case(B: int, H: int, T: int, d: int, seed: int, *, w1_std: float | None = None,
                  **kw):
    """Seeded problem for the two-layer inner model f(x) = W2 silu(W1 x).

    Everything but W1 is ``make_case(B, H, T, d, seed, **kw)``, whose W0 serves
    as W2 (N(0, 0.02^2), the pages' init of the inner weight).  W1 [B,H,d,d] is
    drawn from its own generator, ``PCG64(SeedSequence([seed, 1]))``, as
    N(0, w1_std^2) float32 with w1_std = 1/sqrt(d) by default (a fan-in scale,
    so that W1 k is of order one and the SiLU works in its curved range; the
    pages give no scale for it).  Returns ``(inputs, W1)``."""
    case = make_case(B, H, T, d, seed, **kw)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    std = 1.0 / np.sqrt(d) if w1_std is None else w1_std
    W1 = _f32(rng.standard_normal((B, H, d, d), dtype=np.float32).astype(np.float64) * std)
    case.meta["w1_std"] = std
    return case, W1


def make_mlp_inputs(workload: str, **overrides):
    """A named workload for the two-layer inner model: ``(inputs, W1)``, where
    ``inputs`` is ``make_inputs(workload, **overrides)`` (its W0 serves as W2)
    and W1 is drawn as in ``make_mlp_case`` from the workload's seed."""
    cfg = dict(WORKLOADS[workload])
    cfg.update(overrides)
    B, H, T, d, seed = cfg.pop("B"), cfg.pop("H"), cfg.pop("T"), cfg.pop("d"), cfg.pop("seed")
    return make_mlp_case(B, H, T, d, seed, name=workload, **cfg)
