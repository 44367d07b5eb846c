"""Online-softmax edge cases of the bf16 attention kernel, against the fp64 oracle.

The kernel takes probabilities against a running maximum and raises that
maximum only when a 64-key tile's probabilities would pass 2^16 (then it
rescales O and l and redoes the tile); each KV split keeps its own maximum
until the split-KV combine merges them (GCTStream explainer, "Frame-by-Frame
Causal Processing": the new frame attends over every cached key).  The inputs
here make that branch fire in many tiles and in every split:

- per-frame key scales that grow so that each frame's largest logit passes the
  previous frames' by more than 16 log2 units (logits up to about +-95);
- the same frames in falling order (a large first maximum, later tiles
  underflow against it);
- one dominant key with logit 120 for one query row;

and every split count from 1 to 16.  Outputs are compared with the fp64
oracle at the bf16 tolerance, and the log-sum-exp within LSE_ABS_BF16.  Before
the GPU call, a host count over the same 64-key tiles shows how many tiles
raise the running maximum by more than 16 log2 units after a split's first
tile, so the test fails if the inputs stop reaching the branch.
"""

import numpy as np
import pytest

from bounded_kv_cache_stream_amd import kvstream as kv
from bounded_kv_cache_stream_amd import synth
from oracle import attention
from tests.gpu_common import LSE_ABS_BF16, assert_close, max_abs, say, to64, torch_cuda

pytestmark = pytest.mark.gpu

T, H, D = 200, 2, 64  # 200-token pages: tiles of 64, 64, 64 and 8 keys
LOG2E = 1.4426950408889634


def _raises_after_first_tile(q64, K64, page_lens, splits, tau):
    """Per (query row, head, split): tiles after the split's first whose largest logit passes the running
    maximum by more than 16 log2 units (64-key tiles per page, splits over the tile sequence)."""
    tiles = []
    start = 0
    for n in page_lens:
        for t0 in range(0, n, 64):
            tiles.append((start + t0, start + min(t0 + 64, n)))
        start += n
    count = 0
    for h in range(q64.shape[1]):
        z = (q64[:, h, :] @ K64[:, h, :].T) * tau * LOG2E  # [n_q, N] log2 units
        tmax = np.stack([z[:, a:b].max(axis=1) for a, b in tiles], axis=1)
        for sp in range(splits):
            b, e = sp * len(tiles) // splits, (sp + 1) * len(tiles) // splits
            if e - b < 2:
                continue
            run = np.maximum.accumulate(tmax[:, b:e], axis=1)
            count += int(np.sum(tmax[:, b + 1:e] > run[:, :-1] + 16.0))
    return count


def _cache(frames):
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=1, sliding_window=frames,
                         keyframe_interval=1, pages_per_layer=frames + 2, max_queries=T, max_splits=16)
    return kv.KVCache(cfg, device="cuda")


@pytest.mark.parametrize("order", ["rising", "falling"])
def test_running_max_raised_in_many_tiles_and_splits(order):
    torch = torch_cuda()
    # key scale per frame: logit std ~ alpha, largest logit over a page ~ 2.8 alpha
    alphas = [1.0, 6.0, 11.0, 16.0, 21.0]
    if order == "falling":
        alphas = alphas[::-1]
    F = len(alphas)
    c = _cache(F)
    ks, vs = [], []
    q = synth.iid_frame(120, 0, 0, (T, H, D), device="cuda", dtype=torch.float32)[0]
    for t, a in enumerate(alphas):
        _, k, v = synth.iid_frame(120, 0, t + 1, (T, H, D), device="cuda", dtype=torch.float32)
        k = k * (a / 8.0)
        if t == 2:
            # a dominant key for query row 5 of head 0: logit 120, above every other key of that row
            k[77, 0] = q[5, 0] * (120.0 / float(q[5, 0].pow(2).sum()))
        ks.append(k.to(torch.bfloat16))
        vs.append(v.to(torch.bfloat16))
        c.append(0, t, ks[-1].contiguous(), vs[-1].contiguous())
        c.evict(0)
    qb = q.to(torch.bfloat16).contiguous()
    q64 = to64(qb)
    K64 = np.concatenate([to64(k) for k in ks])
    V64 = np.concatenate([to64(v) for v in vs])
    ref, ref_lse = attention.attend(q64, K64, V64, 1.0)
    logits = np.einsum("qhd,khd->qhk", q64, K64)
    say(f"{order}: logits span {logits.min():.1f} .. {logits.max():.1f}; row 5 head 0 max {logits[5, 0].max():.2f}")
    assert logits.max() > 55.0 and logits.min() < -55.0
    assert logits[5, 0].max() > np.sort(logits[5, 0])[-2] + 15.0
    total = 0
    for splits in (1, 2, 3, 5, 8, 16):
        c.set_splits(splits)
        raises = _raises_after_first_tile(q64, K64, [T] * F, splits, 1.0)
        total += raises
        lse = torch.empty(T * H, dtype=torch.float32, device="cuda")
        out = c.attend(0, qb, 1.0, lse=lse)
        ma, rl = assert_close(to64(out), ref, bf16=True, what=f"{order}, {splits} splits")
        le = max_abs(to64(lse).reshape(T, H), ref_lse)
        assert le <= LSE_ABS_BF16, f"{order}, {splits} splits: LSE off by {le:.3e}"
        # the dominant key's row is its value
        assert np.abs(to64(out)[5, 0] - V64[2 * T + 77, 0]).max() <= 2e-2
        say(f"{order}, {splits} splits: {raises} late max raises on the host count; max_abs {ma:.2e} "
            f"rel_l2 {rl:.2e} lse {le:.2e}")
    if order == "rising":
        assert total >= 1000, total


def test_running_max_raised_at_the_frame1004_shape():
    # 16 heads x 1004-token pages (ragged last tile), 8 frames whose key scales grow by 5 per frame (the
    # largest logit of a row grows by about 16 natural units = 23 log2 units per frame), 1004 queries: the
    # tiles of the headline shape with the branch firing at the frame boundaries inside each split
    torch = torch_cuda()
    Tf, Hf, F = 1004, 16, 8
    cfg = kv.make_config(num_layers=1, num_heads=Hf, page_tokens=Tf, scale_frames=1, sliding_window=F,
                         keyframe_interval=1, pages_per_layer=F + 2, max_queries=Tf, max_splits=16)
    c = kv.KVCache(cfg, device="cuda")
    q = synth.iid_frame(121, 0, 0, (Tf, Hf, D), device="cuda", dtype=torch.float32)[0].to(torch.bfloat16)
    ks, vs = [], []
    for t in range(F):
        _, k, v = synth.iid_frame(121, 0, t + 1, (Tf, Hf, D), device="cuda", dtype=torch.float32)
        ks.append((k * ((1.0 + 5.0 * t) / 8.0)).to(torch.bfloat16))
        vs.append(v.to(torch.bfloat16))
        c.append(0, t, ks[-1].contiguous(), vs[-1].contiguous())
        c.evict(0)
    q64 = to64(q)
    rows = np.random.default_rng(121).choice(Tf, 96, replace=False)
    K64 = np.concatenate([to64(k) for k in ks])
    V64 = np.concatenate([to64(v) for v in vs])
    ref, ref_lse = attention.attend(q64[rows], K64, V64, 1.0)
    for splits in (1, 3, 5):
        c.set_splits(splits)
        raises = _raises_after_first_tile(q64[rows], K64, [Tf] * F, splits, 1.0)
        assert raises >= 1000, (splits, raises)
        lse = torch.empty(Tf * Hf, dtype=torch.float32, device="cuda")
        out = c.attend(0, q.contiguous(), 1.0, lse=lse)
        ma, rl = assert_close(to64(out)[rows], ref, bf16=True, what=f"1004-token pages, {splits} splits")
        le = max_abs(to64(lse).reshape(Tf, Hf)[rows], ref_lse)
        assert le <= LSE_ABS_BF16, f"{splits} splits: LSE off by {le:.3e}"
        say(f"1004-token pages, {splits} splits: {raises} late max raises in the sampled rows; max_abs {ma:.2e} "
            f"rel_l2 {rl:.2e} lse {le:.2e}")
