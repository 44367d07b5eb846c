"""kv_append_attend (one call per frame: page write, eviction, attention) against
the separate calls it stands for.

Two pools see the same frames: one through kv_append_frame -> kv_evict ->
stream_attend, the other through kv_append_attend, whose page write shares the
launch that uploads the attention's page table.  The attention kernel and its
tiles are the same, so outputs and LSE must be equal bit for bit, and so must
eviction counts, page tables and the bytes of every page in the table (K, V,
zero padding and token ids).  Frames are also checked against the fp64
oracle.  Covered: the 1004-token / 16-head stream through the scale phase and
the start of eviction, ragged frames with transient non-keyframes at several
split counts, a one-tile frame, special-token persistence, an fp32 pool, a
diversity-pruned pool (per-head tables built after the upload) and CLCES
compaction of the pages these calls wrote.
"""

import numpy as np
import pytest

from bounded_kv_cache_stream_amd import kvstream as kv
from bounded_kv_cache_stream_amd import synth
from oracle import attention, window
from tests.gpu_common import LSE_ABS_BF16, LSE_ABS_FP32, assert_close, max_abs, say, to64, torch_cuda

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same_pages(a, b, layer, what):
    """Page tables, and the bytes of every page in the table: whole pages (padding and ids included) for
    frame pages, which page writes fill completely; the first len rows of special pages (frame id < 0),
    whose other rows no call writes."""
    torch = a.torch
    ids, lens, frames = a.page_table(layer)
    assert (ids, lens, frames) == b.page_table(layer), f"{what}: page tables differ"
    for pid, n, f in zip(ids, lens, frames):
        for x, y, name in zip(a.page_view(layer, pid), b.page_view(layer, pid), ("K", "V", "ids")):
            if f < 0:
                x, y = (x[:n], y[:n]) if name == "ids" else (x[:, :n], y[:, :n])
            if not torch.equal(_bits(x), _bits(y)):
                rows = (_bits(x) != _bits(y)).reshape(-1, *x.shape[-1:]).any(-1).nonzero().flatten()[:8].tolist() \
                    if name != "ids" else (x != y).nonzero().flatten()[:8].tolist()
                raise AssertionError(f"{what}: {name} of page {pid} (frame {f}, len {n}) differs at {rows}")


class Pair:
    """A pool driven by the separate calls and one driven by kv_append_attend."""

    def __init__(self, cfg, splits=0):
        self.torch = torch_cuda()
        self.cfg = cfg
        self.a = kv.KVCache(cfg, device="cuda")
        self.b = kv.KVCache(cfg, device="cuda")
        if splits:
            self.a.set_splits(splits)
            self.b.set_splits(splits)

    def step(self, t, k, v, q, tau, what):
        torch = self.torch
        n = q.shape[0] * q.shape[1]
        la = torch.empty(n, dtype=torch.float32, device="cuda")
        lb = torch.empty(n, dtype=torch.float32, device="cuda")
        self.a.append(0, t, k, v)
        na = self.a.evict(0)
        oa = self.a.attend(0, q, tau, lse=la)
        ob, nb = self.b.append_attend(0, t, k, v, q, tau, lse=lb)
        assert na == nb, f"{what}: evicted {na} vs {nb}"
        assert torch.equal(_bits(oa), _bits(ob)), f"{what}: outputs differ"
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), f"{what}: lse differs"
        ia, ib = self.a.info(0), self.b.info(0)
        assert ia == ib, f"{what}: info {ia} vs {ib}"
        return ob, lb


# name: tokens, heads, scale frames, window, keyframe interval, special tokens, frames, splits, dtype
CASES = {
    "frame1004_h16_window64": (1004, 16, 8, 64, 1, 0, 76, 0, "bf16"),
    "long_table200": (16, 2, 1, 199, 1, 0, 205, 0, "bf16"),
    "ragged100_kf4": (100, 4, 1, 3, 4, 0, 22, 0, "bf16"),
    "ragged100_kf4_one_split": (100, 4, 1, 3, 4, 0, 22, 1, "bf16"),
    "ragged100_kf4_five_splits": (100, 4, 1, 3, 4, 0, 22, 5, "bf16"),
    "one_tile16": (16, 2, 1, 4, 1, 0, 12, 0, "bf16"),
    "special3": (100, 2, 1, 2, 1, 3, 14, 0, "bf16"),
    "fp32": (16, 2, 1, 4, 1, 0, 12, 0, "fp32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_append_attend_equals_separate_calls(name):
    torch = torch_cuda()
    T, H, S, W, k_int, sp, F, splits, dname = CASES[name]
    dt = torch.bfloat16 if dname == "bf16" else torch.float32
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, dtype=kv.KV_BF16 if dname == "bf16" else kv.KV_FP32,
                         scale_frames=S, sliding_window=W, keyframe_interval=k_int,
                         pages_per_layer=S + W + 1 + (3 if sp else 0), max_queries=max(S, 1) * T, max_splits=16,
                         special_tokens=sp)
    p = Pair(cfg, splits)
    tau = 0.125
    host = {}
    pending = []
    checks = {S - 1, F - 1} | ({71, 72} if F > 72 else set())
    for t in range(F):
        q, k, v = synth.iid_frame(97, 0, t, (T, H, 64), device="cuda", dtype=dt)
        host[t] = (k.double().cpu().numpy(), v.double().cpu().numpy())
        if t < S - 1:
            for c in (p.a, p.b):
                c.append(0, t, k, v)
                c.evict(0)
            pending.append(q)
            continue
        if t == S - 1 and pending:
            q = torch.cat(pending + [q])
        out, lse = p.step(t, k, v, q, tau, f"{name} frame {t}")
        if t in checks:
            att = window.attended_frames(t, S, W, k_int) if not sp else None
            if att is not None:
                K = np.concatenate([host[f][0] for f in att])
                V = np.concatenate([host[f][1] for f in att])
                ref, ref_lse = attention.attend(to64(q), K, V, tau)
                ma, rl = assert_close(to64(out), ref, bf16=dname == "bf16", what=f"{name} frame {t} vs oracle")
                assert max_abs(to64(lse).reshape(ref_lse.shape), ref_lse) <= (LSE_ABS_BF16 if dname == "bf16" else LSE_ABS_FP32)
                say(f"{name} frame {t}: {len(att)} frames attended, max_abs {ma:.2e} rel_l2 {rl:.2e}")
        if t % 4 == 3 or t == F - 1:
            torch.cuda.synchronize()
            _same_pages(p.a, p.b, 0, f"{name} frame {t}")
    if sp:
        info = p.b.info(0)
        assert info["special_pages"] >= 1 and info["special_tokens"] == sp * info["evictions"]


def test_append_attend_pages_then_clces_compaction():
    # CLCES pool: append -> attend -> score_and_compact each frame; compaction
    # moves rows of the pages these calls wrote
    torch = torch_cuda()
    T, H, F, keep = 100, 2, 10, 250
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=0, sliding_window=0,
                         keyframe_interval=1, pages_per_layer=F + 1, max_queries=T, max_splits=8, max_window=5)
    p = Pair(cfg)
    table = torch.from_numpy(synth.raw_scores(98, F * T, 1)).cuda()
    ka = torch.empty(keep, dtype=torch.int32, device="cuda")
    kb = torch.empty(keep, dtype=torch.int32, device="cuda")
    for t in range(F):
        q, k, v = synth.iid_frame(98, 0, t, (T, H, 64), device="cuda", dtype=torch.bfloat16)
        p.step(t, k, v, q, 0.125, f"clces frame {t}")
        na = p.a.score_and_compact(0, table, 5, 0.5, keep, keep_ids=ka)
        nb = p.b.score_and_compact(0, table, 5, 0.5, keep, keep_ids=kb)
        assert na == nb
        torch.cuda.synchronize()
        if na >= keep:
            assert torch.equal(ka, kb), f"clces frame {t}: keep sets differ"
        _same_pages(p.a, p.b, 0, f"clces frame {t}")
    say(f"clces: {F} frames, pages equal after every compaction")


def test_append_attend_on_a_pruned_pool():
    # heads hold different rows after a diversity prune: the per-head tables
    # are built on the device from the shared table the page write uploaded
    torch = torch_cuda()
    T, H, F = 100, 4, 7
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=1, sliding_window=0,
                         keyframe_interval=1, pages_per_layer=F + 1, max_queries=T, max_splits=8, max_window=5)
    p = Pair(cfg)
    for t in range(F):
        q, k, v = synth.iid_frame(99, 0, t, (T, H, 64), device="cuda", dtype=torch.bfloat16)
        if t < 4:
            for c in (p.a, p.b):
                c.append(0, t, k, v)
            continue
        p.step(t, k, v, q, 0.125, f"pruned frame {t}")
        for c in (p.a, p.b):
            c.diversity_score(0)
            c.diversity_prune(0, 150)
        torch.cuda.synchronize()
        assert p.a.head_lengths(0) == p.b.head_lengths(0)
        _same_pages(p.a, p.b, 0, f"pruned frame {t}")


def test_append_attend_errors_change_nothing():
    torch = torch_cuda()
    T, H = 100, 2
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=1, sliding_window=2,
                         keyframe_interval=1, pages_per_layer=4, max_queries=T, max_splits=4)
    c = kv.KVCache(cfg, device="cuda")
    q, k, v = synth.iid_frame(96, 0, 0, (T, H, 64), device="cuda", dtype=torch.bfloat16)
    c.append_attend(0, 0, k, v, q, 0.125)
    before = (c.page_table(0), c.info(0))
    with pytest.raises(kv.KVError) as e:  # frame order
        c.append_attend(0, 0, k, v, q, 0.125)
    assert e.value.status == kv.KV_ERR_STATE
    with pytest.raises(kv.KVError) as e:  # bad scale
        c.append_attend(0, 1, k, v, q, 0.0)
    assert e.value.status == kv.KV_ERR_ARG
    with pytest.raises(kv.KVError) as e:  # too many queries
        c.append_attend(0, 1, k, v, torch.cat([q, q]), 0.125)
    assert e.value.status == kv.KV_ERR_SHAPE
    with pytest.raises(ValueError):  # V shorter than K: refused before any call (it would be read past its end)
        c.append_attend(0, 1, k, v[:50].contiguous(), q, 0.125)
    with pytest.raises(ValueError):
        c.append(0, 1, k, v[:50].contiguous())
    assert (c.page_table(0), c.info(0)) == before
    # the pool needs S + W + 1 = 4 page ids: with 3, the fourth keyframe finds none
    small = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=1, sliding_window=2,
                           keyframe_interval=1, pages_per_layer=3, max_queries=T, max_splits=4)
    s = kv.KVCache(small, device="cuda")
    for t in range(3):
        s.append_attend(0, t, k, v, q, 0.125)
    before = (s.page_table(0), s.info(0))
    with pytest.raises(kv.KVError) as e:
        s.append_attend(0, 3, k, v, q, 0.125)
    assert e.value.status == kv.KV_ERR_NO_PAGES
    assert (s.page_table(0), s.info(0)) == before
    torch.cuda.synchronize()
