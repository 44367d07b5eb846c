"""Softmax attention of a frame's queries over the retained cache, in float64.

Oracle (test infrastructure only).  Sources: GCTStream explainer ("How
GCTStream Implements Streaming 3D Reconstruction with KV Cache"), section
"Frame-by-Frame Causal Processing" (each new frame attends to the cached keys
and values of earlier frames) and section "Scale-Frame Phase" (the first frames
are processed together with bidirectional attention); InfiniteVGGT explainer,
"Causal Attention" (store past keys/values, the new frame queries them).

Definition, per head ``h`` (no token mask: causality is between frames, a
frame sees all of its own tokens):

    Z   = tau * Q_h K_h^T
    m   = max_j Z[:, j]
    P   = exp(Z - m)
    l   = sum_j P[:, j]
    O_h = (P V_h) / l
    LSE = m + ln(l)

The inputs are the exact values the GPU receives (bf16 or fp32), widened to
float64.  Rows of ``Q`` are independent, so they may be processed in chunks to
bound memory; no reduction is split or reordered beyond the library matmul.

Pinned by ``tests/test_oracle_attention.py``: brute-force dense attention with
a frame mask over the whole stream, rows summing to one, V = 1 gives 1,
Q = 0 gives mean(V), one key gives its value, permutation invariance of the
cache order, linearity in V, and a two-token example worked by hand.
"""

from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float,
           row_chunk: int = 256) -> tuple[np.ndarray, np.ndarray]:
    """Attention of ``q [n_q, H, D]`` over ``k, v [N, H, D]``.

    Returns ``(out [n_q, H, D] float64, lse [n_q, H] float64)``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, H, D = q.shape
    N = k.shape[0]
    if k.shape != (N, H, D) or v.shape != (N, H, D):
        raise ValueError("k and v must be [N, H, D] with the query's H and D")
    if N == 0:
        raise ValueError("attention over an empty cache is undefined")
    out = np.empty((n_q, H, D), dtype=np.float64)
    lse = np.empty((n_q, H), dtype=np.float64)
    for h in range(H):
        kh = np.ascontiguousarray(k[:, h, :])
        vh = np.ascontiguousarray(v[:, h, :])
        for r0 in range(0, n_q, row_chunk):
            qh = q[r0:r0 + row_chunk, h, :]
            z = tau * (qh @ kh.T)
            m = z.max(axis=1, keepdims=True)
            p = np.exp(z - m)
            l = p.sum(axis=1, keepdims=True)
            out[r0:r0 + row_chunk, h, :] = (p @ vh) / l
            lse[r0:r0 + row_chunk, h] = (m + np.log(l))[:, 0]
    return out, lse


def gather_frames(frames: dict, order: list[int]) -> np.ndarray:
    """Concatenate per-frame ``[T, H, D]`` arrays in the given logical order."""
    return np.concatenate([np.asarray(frames[f]) for f in order], axis=0)


def gather_tokens(token_rows, token_ids: list[int] | np.ndarray, tokens_per_frame: int) -> np.ndarray:
    """Rows ``[len(ids), H, D]`` of global token ids ``frame * T + slot``.

    ``token_rows(frame)`` returns that frame's ``[T, H, D]`` array.
    """
    ids = np.asarray(token_ids, dtype=np.int64)
    frames = ids // tokens_per_frame
    slots = ids % tokens_per_frame
    first = np.asarray(token_rows(int(frames[0])))
    out = np.empty((len(ids),) + first.shape[1:], dtype=first.dtype)
    for f in np.unique(frames):
        sel = frames == f
        out[sel] = np.asarray(token_rows(int(f)))[slots[sel]]
    return out
