"""Seeded synthetic inputs for the five streaming workloads.

This module holds input generation only -- shapes, seeds and the random
recipes -- and none of the cache or attention arithmetic.  The tests and the
benchmark feed the same generated arrays to the HIP library and to the CPU
oracle.

Recipes (the pages measure on recorded video; these stand in for it):

* frame shape: 518x378 pixels with 14-pixel patches is 37x27 = 999 patch
  tokens plus 5 special tokens = 1004 tokens per frame, 16 heads x 64 dims
  (LingBot-Map 20 FPS explainer, opening claim on 518x378 frames);
* slow camera motion: every Q/K/V tensor follows the AR(1) recurrence
  ``X_0 = e_0``, ``X_t = 0.7 X_{t-1} + 0.3 e_t`` with ``e_t ~ N(0, 1)``, kept in
  fp32; Q is passed as ``X^Q / sqrt(64)``; bf16 rounding happens only on the
  copy handed over (InfiniteVGGT explainer, "The Gap": consecutive frames are
  near-duplicates);
* raw CLCES scores: the L2 norm of a synthetic FFN residual
  ``r ~ N(0, u I_1024)`` with a per-token scale ``u ~ LogNormal(0, 0.5)``,
  drawn in the equivalent form ``s = sqrt(u * chi2_1024)`` (StreamCacheVGGT
  article, 2.1.1: the raw score is the L2 norm of the FFN residual).

Every draw is keyed by ``(workload, layer, stream, frame)``; streams are
0/1/2 = Q/K/V, 3 = raw scores, 4 = the per-token scale ``u``.
"""

from __future__ import annotations

import numpy as np

Q_STREAM, K_STREAM, V_STREAM, SCORE_STREAM, SCALE_STREAM = 0, 1, 2, 3, 4

TOKENS_PER_FRAME = 1004  # 37 * 27 patch tokens + 5 special tokens

WORKLOADS = {
    0: dict(name="tiny_fp32_t16_h2_s1_w4_k1", dtype="fp32", layers=1, heads=2, head_dim=64,
            tokens=16, scale_frames=1, window=4, keyframe_interval=1, frames=12,
            sm_scale=0.125, ar1=False),
    1: dict(name="frame1004_h16_d64_s8_w64_k1_f200", dtype="bf16", layers=1, heads=16, head_dim=64,
            tokens=TOKENS_PER_FRAME, scale_frames=8, window=64, keyframe_interval=1, frames=200,
            sm_scale=1.0, ar1=True),
    2: dict(name="frame1004_h16_d64_s8_w64_k4_f10000", dtype="bf16", layers=1, heads=16, head_dim=64,
            tokens=TOKENS_PER_FRAME, scale_frames=8, window=64, keyframe_interval=4, frames=10000,
            sm_scale=1.0, ar1=True),
    3: dict(name="clces_l24_n72288_w5_lam0.5_keep50", dtype="bf16", layers=24, heads=16, head_dim=64,
            tokens=TOKENS_PER_FRAME, cache_frames=72, clces_window=5, lam=0.5, keep=36144,
            scale_frames=0, window=0, keyframe_interval=1, sm_scale=1.0, ar1=False),
    4: dict(name="budget_l24_h16_d64_b128512_f500", dtype="bf16", layers=24, heads=16, head_dim=64,
            tokens=TOKENS_PER_FRAME, budget=128512, frames=500, clces_window=5, lam=0.5,
            scale_frames=0, window=0, keyframe_interval=1, sm_scale=1.0, ar1=True),
}


def seed(workload: int, layer: int, stream: int, frame: int) -> int:
    """64-bit seed for one draw, from numpy's SeedSequence."""
    st = np.random.SeedSequence([workload, layer, stream, frame]).generate_state(2, dtype=np.uint32)
    return (int(st[0]) | (int(st[1]) << 32)) & 0x7FFF_FFFF_FFFF_FFFF


def _normal(torch, shape, s: int, device):
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def iid_frame(workload: int, layer: int, frame: int, shape, device="cpu", dtype=None):
    """``(q, k, v)``, each ``N(0, 1)`` of ``shape``, in ``dtype`` (default fp32)."""
    import torch
    dtype = dtype or torch.float32
    return tuple(_normal(torch, shape, seed(workload, layer, st, frame), device).to(dtype)
                 for st in (Q_STREAM, K_STREAM, V_STREAM))


class AR1Stream:
    """Frame-correlated Q/K/V of one layer: ``X_t = 0.7 X_{t-1} + 0.3 e_t`` (fp32 state)."""

    RHO = 0.7
    NOISE = 0.3

    def __init__(self, workload: int, layer: int, shape, device="cpu", q_scale: float = 0.125):
        import torch
        self.torch = torch
        self.workload = workload
        self.layer = layer
        self.shape = tuple(shape)
        self.device = device
        self.q_scale = q_scale
        self.state = None
        self.frame = -1

    def next(self):
        """Advance one frame; returns bf16 ``(q, k, v)`` on the stream's device."""
        torch = self.torch
        self.frame += 1
        eps = [_normal(torch, self.shape, seed(self.workload, self.layer, st, self.frame), self.device)
               for st in (Q_STREAM, K_STREAM, V_STREAM)]
        if self.state is None:
            self.state = eps
        else:
            self.state = [self.RHO * x + self.NOISE * e for x, e in zip(self.state, eps)]
        xq, xk, xv = self.state
        return ((xq * self.q_scale).to(torch.bfloat16), xk.to(torch.bfloat16), xv.to(torch.bfloat16))


def raw_scores(workload: int, n_tokens: int, n_layers: int, dim: int = 1024) -> np.ndarray:
    """Raw score table ``[n_tokens, n_layers]`` fp32, row = global token id."""
    rng_u = np.random.default_rng(seed(workload, 0, SCALE_STREAM, 0))
    u = rng_u.lognormal(mean=0.0, sigma=0.5, size=n_tokens)
    out = np.empty((n_tokens, n_layers), dtype=np.float32)
    for l in range(n_layers):
        rng = np.random.default_rng(seed(workload, l, SCORE_STREAM, 0))
        chi2 = rng.chisquare(dim, size=n_tokens)
        out[:, l] = np.sqrt(u * chi2).astype(np.float32)
    return out
