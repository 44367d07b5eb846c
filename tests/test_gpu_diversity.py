"""GPU parity of the diversity-scored per-head prune (InfiniteVGGT explainer).

Scores: float64 on both sides, equal within SCORE_ABS (the two add the
normalised keys in different orders).  The top-K decision is taken on the
float64 scores on both sides; each compared prune first checks that the
oracle's K-th and (K+1)-th scores are either exactly equal (an exact tie,
which both sides break by candidate index) or further apart than the score
bound, so that the keep set is unique, and then keep sets, per-head page
lengths, released pages and the bytes of every compacted page are compared
bit-exactly.  Attention over the per-head pages a prune leaves is compared
within the bf16 / fp32 tolerance.
"""

import numpy as np
import pytest

from bounded_kv_cache_stream_amd import kvstream as kv
from bounded_kv_cache_stream_amd import synth
from oracle import attention, clces, diversity
from tests.gpu_common import assert_close, say, to64, torch_cuda

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": kv.KV_BF16, "fp32": kv.KV_FP32}


def _cfg(T, pages, H, dtype, layers=1, max_queries=None):
    # scale_frames = 1: frame 0 is the anchor, never a candidate
    return kv.make_config(num_layers=layers, num_heads=H, page_tokens=T, dtype=dtype, scale_frames=1,
                          sliding_window=0, keyframe_interval=1, pages_per_layer=pages,
                          max_queries=max_queries or T, max_splits=8, max_window=5)


# The kernel adds the normalised keys in another order than the oracle (pages,
# then blocks of rows) and divides once by |k||S| instead of normalising each
# key first, so the float64 scores differ by rounding only: up to ~1e-14 in
# absolute terms (8.4e-15 over 16 heads x 128,512 keys when the kernel's
# summation order is replayed in numpy).  Scores lie in [-1, 1].
SCORE_ABS = 1e-13


def _assert_scores(gpu, ref64, what):
    """gpu, ref64: float64 [n] scores of the kernel and the oracle; returns the largest difference."""
    err = float(np.max(np.abs(gpu - ref64))) if len(gpu) else 0.0
    assert err <= SCORE_ABS, f"{what}: score off by {err:.3e}"
    return err


def _assert_decided(ref64, k, what):
    """The top-k of the oracle's scores is unique: the k-th and (k+1)-th largest are exactly equal (both
    sides break the tie by index) or more than twice the score bound apart."""
    if 0 < k < len(ref64):
        srt = np.sort(ref64)[::-1]
        gap = srt[k - 1] - srt[k]
        assert gap == 0.0 or gap > 2 * SCORE_ABS, f"{what}: threshold gap {gap:.3e} within the score bound"


class Stream:
    """One layer of H heads: host copies of every appended frame, the oracle cache and the GPU cache."""

    def __init__(self, cache, T, H, pages, wid, layer=0):
        self.cache, self.T, self.H, self.layer, self.wid = cache, T, H, layer, wid
        self.frames = {}
        self.sim = diversity.DiversityCache(H, T, pages)
        self.torch = cache.torch
        self.dt = self.torch.bfloat16 if cache.cfg.dtype == kv.KV_BF16 else self.torch.float32

    def append(self, t, k=None, v=None):
        if k is None:
            _, k, v = synth.iid_frame(self.wid, self.layer, t, (self.T, self.H, 64), device="cuda", dtype=self.dt)
        self.cache.append(self.layer, t, k, v)
        self.frames[t] = (k.cpu(), v.cpu())
        self.sim.append(t)

    def key_of(self, f, h):
        return self.frames[f][0][:, h, :].double().numpy()

    def prune(self, k):
        """The oracle's prune to k per head, once each head's top-k is shown to be unique."""
        for h, sc in enumerate(self.sim.scores(self.key_of)):
            _assert_decided(sc, k, f"layer {self.layer} head {h}")
        return self.sim.prune(self.key_of, k)

    def check_pages(self, what):
        """Page table, per-head lengths and the first n_h rows of K and V of every page and head, bit-exact."""
        torch = self.torch
        ids, _, frames = self.cache.page_table(self.layer)
        hl = self.cache.head_lengths(self.layer)
        want = self.sim.page_table()
        assert [(p, f, tuple(n)) for p, f, n in zip(ids, frames, hl)] == want, what
        for pid, f, per_head in self.sim.table:
            k, v, _ = self.cache.page_view(self.layer, pid)
            for h in range(self.H):
                n = len(per_head[h])
                fr, sl = per_head[h] // self.T, per_head[h] % self.T
                ek = torch.stack([self.frames[int(a)][0][int(b), h] for a, b in zip(fr, sl)]) if n else None
                ev = torch.stack([self.frames[int(a)][1][int(b), h] for a, b in zip(fr, sl)]) if n else None
                if n:
                    bits = torch.int16 if self.dt == torch.bfloat16 else torch.int32
                    assert torch.equal(k[h, :n].cpu().view(bits), ek.view(bits)), f"{what}: K page {pid} head {h}"
                    assert torch.equal(v[h, :n].cpu().view(bits), ev.view(bits)), f"{what}: V page {pid} head {h}"

    def check_attention(self, q, tau, what):
        # every KV tiling of the per-head tables (the automatic choice, tiles per page, tiles packed across
        # page ends) against the same oracle
        outs = []
        for tiling in (kv.KV_TILING_AUTO, kv.KV_TILING_PAGE, kv.KV_TILING_PACKED):
            self.cache.set_tiling(tiling)
            outs.append((tiling, self.cache.attend(self.layer, q, tau)))
        self.cache.set_tiling(kv.KV_TILING_AUTO)
        ref = np.empty(tuple(q.shape), dtype=np.float64)
        q64 = to64(q)
        for h in range(self.H):
            ids = self.sim.all_ids(h)
            K = attention.gather_tokens(lambda f: self.frames[f][0][:, h:h + 1].double().numpy(), ids, self.T)
            V = attention.gather_tokens(lambda f: self.frames[f][1][:, h:h + 1].double().numpy(), ids, self.T)
            ref[:, h:h + 1], _ = attention.attend(q64[:, h:h + 1], K, V, tau)
        for tiling, out in outs:
            assert_close(to64(out), ref, bf16=self.dt == self.torch.bfloat16, what=f"{what} (tiling {tiling})")


@pytest.mark.parametrize("dname", ["bf16", "fp32"])
def test_diversity_small_ragged(dname):
    # 4 heads, 100 tokens per frame (a ragged last tile), 8 frames.  Head 0 of
    # frame 2 holds one direction only, so it dominates that head's mean and
    # scores lowest: the prune empties that page in head 0 only, which leaves
    # a zero-length entry in head 0's attention table.  One key is zero.
    torch = torch_cuda()
    T, H, F, K = 100, 4, 8, 450
    dt = torch.bfloat16 if dname == "bf16" else torch.float32
    cache = kv.KVCache(_cfg(T, F + 1, H, DTYPES[dname]), device="cuda")
    s = Stream(cache, T, H, F + 1, wid=95)
    for t in range(F):
        _, k, v = synth.iid_frame(95, 0, t, (T, H, 64), device="cuda", dtype=torch.float32)
        if t == 2:
            u = torch.ones(64, device="cuda") / 8.0
            k[:, 0, :] = u + 0.01 * k[:, 0, :]
        if t == 3:
            k[5, 1, :] = 0.0
        s.append(t, k.to(dt).contiguous(), v.to(dt).contiguous())
    stride = (F - 1) * T + 3
    sc = torch.full((H, stride), -7.0, dtype=torch.float64, device="cuda")
    mean = cache.diversity_score(0, scores=sc)
    ref = s.sim.scores(s.key_of)
    for h in range(H):
        _assert_scores(sc[h, :len(ref[h])].cpu().numpy(), ref[h], f"head {h}")
        assert np.all(sc[h, len(ref[h]):].cpu().numpy() == -7.0)
    assert abs(mean - s.sim.mean_diversity(s.key_of)) <= 1e-12
    assert sc[1, 2 * T + 5].item() == 0.0  # the zero key (frame 3, slot 5 of head 1)
    kept = cache.diversity_prune(0, K, scores=sc)
    assert kept == [K] * H
    masks = s.prune(K)
    assert not masks[0][T:2 * T].any() and all(m[T:2 * T].any() for m in masks[1:])
    s.check_pages(f"{dname} prune")
    assert cache.info(0)["prunes"] == 1
    q = synth.iid_frame(96, 0, 0, (T, H, 64), device="cuda", dtype=dt)[0] * 0.125
    s.check_attention(q.contiguous(), 1.0, f"{dname} attention after the prune")
    # CLCES refuses a layer whose heads hold different tokens
    with pytest.raises(kv.KVError) as e:
        cache.score_and_compact(0, torch.ones((F * T, 1), device="cuda"), 5, 0.5, 10)
    assert e.value.status == kv.KV_ERR_STATE
    # a second prune to 180 per head, then the per-head page merge: pages 2 and 3 go after page 1 (page 2
    # holds no row of head 0), pages 5 and 6 after page 4, as in the oracle
    assert cache.diversity_prune(0, 180) == [180] * H
    s.prune(180)
    moves = s.sim.merge_pages()
    assert [(m[0], m[1]) for m in moves] == [(2, 1), (3, 1), (5, 4), (6, 4)]
    assert cache.merge_pages(0) == len(moves)
    assert cache.info(0)["merges"] == len(moves)
    s.check_pages(f"{dname} per-head merge")
    s.check_attention(q.contiguous(), 1.0, f"{dname} attention after the merge")
    assert cache.merge_pages(0) == 0


def test_diversity_stream_with_page_merge():
    # per frame: append, prune to 260 per head, per-head page merge; pages, per-head lengths and attention
    # against the oracle every frame (merges start at frame 6)
    torch = torch_cuda()
    T, H, F, B = 100, 4, 14, 260
    cache = kv.KVCache(_cfg(T, F + 1, H, kv.KV_BF16), device="cuda")
    s = Stream(cache, T, H, F + 1, wid=94)
    merged = 0
    for t in range(F):
        s.append(t)
        cache.diversity_prune(0, B)
        s.prune(B)
        n = cache.merge_pages(0)
        moves = s.sim.merge_pages()
        assert n == len(moves), t
        merged += n
        s.check_pages(f"stream frame {t}")
        q = synth.iid_frame(93, 0, t, (T, H, 64), device="cuda", dtype=torch.bfloat16)[0]
        s.check_attention(q, 0.125, f"stream frame {t}")
    assert merged > 0 and cache.info(0)["merges"] == merged
    say(f"diversity stream with page merge: {merged} merges, {len(cache.page_table(0)[0])} pages at the end")


def test_merge_pages_layers_batched():
    # one call merges three layers: layers 0 and 1 are pruned (per-head merges), layer 2 is not (its full
    # pages never fit together); each layer against its own oracle every frame
    torch = torch_cuda()
    T, H, F = 100, 4, 12
    cache = kv.KVCache(_cfg(T, F + 1, H, kv.KV_BF16, layers=3), device="cuda")
    streams = [Stream(cache, T, H, F + 1, wid=92, layer=l) for l in range(3)]
    budgets = (230, 300)
    merged = [0, 0, 0]
    for t in range(F):
        for s in streams:
            s.append(t)
        for l, b in enumerate(budgets):
            cache.diversity_prune(l, b)
            streams[l].prune(b)
        n = cache.merge_pages_layers(0, 3)
        for l in range(3):
            assert n[l] == len(streams[l].sim.merge_pages()), (t, l)
            merged[l] += n[l]
            streams[l].check_pages(f"batched merge frame {t} layer {l}")
    assert merged[0] > 0 and merged[1] > 0 and merged[2] == 0
    q = synth.iid_frame(91, 0, 0, (T, H, 64), device="cuda", dtype=torch.bfloat16)[0]
    for s in streams:
        s.check_attention(q, 0.125, f"after batched merges, layer {s.layer}")


def test_diversity_edge_cases():
    torch = torch_cuda()
    T, H = 64, 2
    cache = kv.KVCache(_cfg(T, 8, H, kv.KV_BF16, layers=3), device="cuda")
    streams = [Stream(cache, T, H, 8, wid=97, layer=l) for l in range(3)]
    for l, s in enumerate(streams):
        for t in range(5):
            _, k, v = synth.iid_frame(97, l, t, (T, H, 64), device="cuda", dtype=torch.float32)
            if l == 1:
                k[:, 1, :] = 0.0  # every key of head 1 is zero: its mean is zero, every score 0
            s.append(t, k.to(torch.bfloat16).contiguous(), v.to(torch.bfloat16).contiguous())
    # a NaN key: error, nothing changes
    k, v, _ = cache.page_view(2, 3)
    saved = k[1, 7, 3].clone()
    k[1, 7, 3] = float("nan")
    with pytest.raises(kv.KVError) as e:
        cache.diversity_prune(2, 10)
    assert e.value.status == kv.KV_ERR_NAN
    with pytest.raises(kv.KVError) as e:
        cache.diversity_score(2)
    assert e.value.status == kv.KV_ERR_NAN
    assert cache.head_lengths(2) == [[T, T]] * 5
    k[1, 7, 3] = saved
    streams[2].check_pages("after the NaN refusal")
    # zero mean in head 1: ties everywhere, the first K candidates stay
    assert cache.diversity_prune(1, 100) == [100, 100]
    streams[1].prune(100)
    assert [n[1] for n in cache.head_lengths(1)] == [T, T, 100 - T, 0, 0]
    streams[1].check_pages("zero mean")
    # keep 0: every candidate page goes, the anchor stays
    assert cache.diversity_prune(0, 0) == [0, 0]
    streams[0].prune(0)
    assert cache.page_table(0)[0] == [0]
    assert cache.info(0)["pages_free"] == 7
    streams[0].check_pages("keep 0")
    q = synth.iid_frame(98, 0, 0, (T, H, 64), device="cuda", dtype=torch.bfloat16)[0]
    streams[0].check_attention(q, 0.125, "anchor only")
    # score stride too small
    with pytest.raises(kv.KVError) as e:
        cache.diversity_score(2, scores=torch.empty((H, 10), dtype=torch.float64, device="cuda"))
    assert e.value.status == kv.KV_ERR_SHAPE


def test_diversity_select_with_more_ties_than_the_lds_list():
    # head 0: every key zero, so every score ties (0) at all 64 bits and more keys match each fixed prefix
    # (8192) than the select's LDS list holds: every pass scans the key planes.  Head 1: iid keys (the list
    # path).  The first K candidates of head 0 stay, in candidate order
    torch = torch_cuda()
    T, H, F = 1024, 2, 9
    cache = kv.KVCache(_cfg(T, F + 1, H, kv.KV_BF16), device="cuda")
    s = Stream(cache, T, H, F + 1, wid=95)
    for t in range(F):
        _, k, v = synth.iid_frame(95, 0, t, (T, H, 64), device="cuda", dtype=torch.float32)
        k[:, 0, :] = 0.0
        s.append(t, k.to(torch.bfloat16).contiguous(), v.to(torch.bfloat16).contiguous())
    assert cache.diversity_prune(0, 5000) == [5000, 5000]
    s.prune(5000)
    s.check_pages("ties beyond the LDS list")
    assert [n[0] for n in cache.head_lengths(0)] == [T, T, T, T, T, 5000 - 4 * T, 0, 0, 0]


@pytest.mark.parametrize("dname", ["bf16", "fp32"])
def test_diversity_stream_every_frame(dname):
    # per frame: append -> attend over the per-head pages -> prune to a fixed
    # per-head budget; pages pruned before are pruned again with their
    # per-head lengths, and new pages join with full heads
    torch = torch_cuda()
    T, H, F, K = 80, 4, 14, 300
    dt = torch.bfloat16 if dname == "bf16" else torch.float32
    cache = kv.KVCache(_cfg(T, F + 1, H, DTYPES[dname]), device="cuda")
    s = Stream(cache, T, H, F + 1, wid=99)
    ar = synth.AR1Stream(99, 0, (T, H, 64), device="cuda")
    for t in range(F):
        q, k, v = ar.next()
        s.append(t, k.to(dt).contiguous(), v.to(dt).contiguous())
        s.check_attention(q.to(dt).contiguous(), 1.0, f"{dname} frame {t}")
        cand = [len(s.sim.candidates(h)) for h in range(H)]
        sc = torch.zeros((H, max(max(cand), 1)), dtype=torch.float64, device="cuda")
        kept = cache.diversity_prune(0, K, scores=sc)
        assert kept == [min(K, n) for n in cand], t
        if max(cand) > K:
            ref = s.sim.scores(s.key_of)
            for h in range(H):
                _assert_scores(sc[h, :cand[h]].cpu().numpy(), ref[h], f"frame {t} head {h}")
        s.prune(K)
        s.check_pages(f"{dname} frame {t}")
    hl = np.array(cache.head_lengths(0))
    assert (hl[1:].sum(axis=0) == K).all() and len(set(map(tuple, hl[1:]))) > 1


def test_diversity_budgets_three_layers():
    # the whole step with the batched calls: mean diversity of every layer
    # (one wait), softmax budgets, prune of every layer (one wait, reusing
    # the keys of the scoring)
    torch = torch_cuda()
    T, H, F, L = 128, 4, 6, 3
    cache = kv.KVCache(_cfg(T, F + 1, H, kv.KV_BF16, layers=L), device="cuda")
    streams = [Stream(cache, T, H, F + 1, wid=100, layer=l) for l in range(L)]
    for l, s in enumerate(streams):
        ar = synth.AR1Stream(100, l, (T, H, 64), device="cuda")
        for t in range(F):
            _, k, v = ar.next()
            if l == 2:
                k = (k.float() + 2.0 * (l + 1)).to(torch.bfloat16)  # a shared offset: low diversity
            s.append(t, k.contiguous(), v)
    means = cache.diversity_score_layers(0, L)
    assert means == [cache.diversity_score(l) for l in range(L)]  # same kernels, same order: same bits
    want = [s.sim.mean_diversity(s.key_of) for s in streams]
    assert np.allclose(means, want, rtol=0, atol=1e-12), (means, want)
    assert means[2] < min(means[:2])
    total = 3 * H * 400
    budgets = kv.kv_layer_budgets(means, 0.1, total, H)
    assert budgets == diversity.layer_budgets(want, 0.1, total, H).tolist()
    kept = cache.diversity_prune_layers(0, budgets)
    for l, s in enumerate(streams):
        assert kept[l] == [min(budgets[l], len(s.sim.candidates(h))) for h in range(H)]
        s.prune(budgets[l])
        s.check_pages(f"layer {l}")
    say(f"budgets {budgets} from mean diversity {np.round(means, 5).tolist()}")
    # unchanged layers: a second batched prune to the same budgets moves nothing
    assert cache.diversity_prune_layers(0, budgets) == kept
    for s in streams:
        s.check_pages("second prune")


def test_diversity_batched_prune_all_or_nothing():
    # a key that is not finite in one layer: the batched prune scores every
    # layer before any row moves, so no layer changes
    torch = torch_cuda()
    T, H, F, L = 64, 2, 5, 3
    cache = kv.KVCache(_cfg(T, F + 1, H, kv.KV_BF16, layers=L), device="cuda")
    streams = [Stream(cache, T, H, F + 1, wid=102, layer=l) for l in range(L)]
    for s in streams:
        for t in range(F):
            s.append(t)
    k, _, _ = cache.page_view(2, 4)
    k[0, 3, 9] = float("inf")
    with pytest.raises(kv.KVError) as e:
        cache.diversity_prune_layers(0, [100, 100, 100])
    assert e.value.status == kv.KV_ERR_NAN and "layer 2" in str(e.value)
    with pytest.raises(kv.KVError) as e:
        cache.diversity_score_layers(0, L)
    assert e.value.status == kv.KV_ERR_NAN and "layer 2" in str(e.value)
    for s in streams[:2]:
        s.check_pages("after the refused prune")
    assert all(cache.head_lengths(l) == [[T, T]] * F for l in range(L))
    # the first two layers alone prune normally
    cache.diversity_prune_layers(0, [100, 100])
    for s in streams[:2]:
        s.prune(100)
        s.check_pages("after the prune of layers 0-1")


def test_diversity_full_size_16_heads():
    # 16 heads x 1004 tokens, 129 frames (the anchor plus 128 candidate pages
    # = 128,512 candidates per head), pruned to 64,256 per head: scores of
    # every candidate, keep sets of every head, and sampled pages bit-exact
    torch = torch_cuda()
    T, H, F, K = synth.TOKENS_PER_FRAME, 16, 129, 64256
    cache = kv.KVCache(_cfg(T, F + 1, H, kv.KV_BF16, max_queries=T), device="cuda")
    ar = synth.AR1Stream(101, 0, (T, H, 64), device="cuda")
    keys = []
    for t in range(F):
        _, k, v = ar.next()
        cache.append(0, t, k, v)
        keys.append(k.cpu())
    N = (F - 1) * T
    sc = torch.empty((H, N), dtype=torch.float64, device="cuda")
    mean = cache.diversity_score(0, scores=sc)
    allk = torch.stack(keys[1:]).double().numpy()  # [F-1, T, H, D]
    ref = [diversity.diversity_scores(allk[:, :, h, :].reshape(N, 64)) for h in range(H)]
    worst = max(_assert_scores(sc[h].cpu().numpy(), ref[h], f"head {h}") for h in range(H))
    assert abs(mean - float(np.mean(np.concatenate(ref)))) <= 1e-12
    say(f"full size: {H}x{N} float64 scores, largest difference from the oracle {worst:.2e}")
    for h in range(H):
        _assert_decided(ref[h], K, f"head {h}")
    sc2 = torch.empty((H, N), dtype=torch.float64, device="cuda")
    assert cache.diversity_prune(0, K, scores=sc2) == [K] * H
    assert torch.equal(sc, sc2)
    hl = np.array(cache.head_lengths(0))
    for h in range(H):
        keep = diversity.topk_desc(ref[h], K).reshape(F - 1, T)
        assert hl[1:, h].tolist() == keep.sum(axis=1).tolist(), f"page lengths of head {h}"
        for p in (0, 37, 127):
            new = clces.compact_page(np.arange(T), keep[p])
            kpage, _, _ = cache.page_view(0, p + 1)
            want = keys[p + 1][new, h]
            assert torch.equal(kpage[h, :len(new)].cpu().view(torch.int16), want.view(torch.int16)), (h, p)
    say(f"full size: {K} kept per head, page lengths of every head and sampled pages bit-exact")
